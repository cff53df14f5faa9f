// Entry points of decode attention: the int8 cache ([P3] Sec. 1-2), the
// integer partials export, and the mixed int4 / int8 cache of the group
// variant ([P4] Sec. 3.2-3.3).  The pipeline itself lives in
// kvq_decode_core.h and is compiled once, here.
#include <atomic>
#include <mutex>

#include "kvq_decode_core.h"
#include "kvq_decode_group.h"

namespace kvq {

// Integer block partials of every (sequence, query head, token): a workgroup
// per (sequence, kv-head, 4 tiles of 64 tokens) runs the decode kernel's
// query quantization, tile loader and matrix-core dot products.
template <bool BS8>
__global__ __launch_bounds__(kWGThreads) void kvq8_qk_partials_kernel(DecodeArgs a, int32_t* __restrict__ partials,
                                                                      int n_groups) {
    __shared__ QSmem qsm;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int m = lane & 15;
    const int G = a.nq / a.nkv;
    const int grp = blockIdx.x % n_groups;
    const int kh = (blockIdx.x / n_groups) % a.nkv;
    const int b = blockIdx.x / (n_groups * a.nkv);
    const float4 qx = load_q4(a.q + ((size_t)b * a.nq + (size_t)kh * G) * kHD, G);
    const int L = effective_len(a.r8, b, a.log2_bs);
    if (grp * kChunkUnit >= L) return;                    // uniform per workgroup
    const int base = (grp * kWaves + wave) * kTile;
    const int32_t* btb = a.r8.bt + (size_t)b * a.r8.max_blocks;
    const int raw = mtile_raw(a.r8, btb, base, a.log2_bs, lane);
    const LaneOff lo = lane_offsets(a, lane, kh);
    MTile T;
    mtile_issue<BS8, kIssueKeys>(a, raw, base, kh, lane, lo, T);
    quantize_q4(qx, G, qsm);
    lds_barrier();
    const MQuery Q = load_q_operand(qsm, G, g, m);
    v4i_t d[4][2];
    mtile_qk(T, Q, d);
    const int H = m >> 1;
    if (H >= G) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int id0 = __builtin_amdgcn_readlane(T.id, 16 * v);
        const int id1 = __builtin_amdgcn_readlane(T.id, 16 * v + 8);
        const int id = (g & 2) ? id1 : id0;          // block of tokens 16v + 4g + r
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = base + 16 * v + 4 * g + r;
                if (t < L && id >= 0)
                    partials[(((size_t)b * a.nq + (size_t)kh * G + H) * a.r8.max_len + t) * 4 + 2 * h + (m & 1)] =
                        d[v][h][r];
            }
    }
}

}  // namespace kvq

using namespace kvq;

extern "C" int kvq8_decode_chunk_tokens(int batch, int nkv, int max_ctx_len) {
    if (batch < 0 || nkv < 1 || max_ctx_len < 0) return 0;
    // up to 2048 tokens per workgroup (longer chunks fill fewer workgroups
    // and leave a longer tail; at most 8 tiles per wave)
    return default_tiles_per_wave((long)batch * nkv, max_ctx_len, 8) * kChunkUnit;
}

static int resolve_chunk8(int batch, int nkv, int max_ctx_len, int chunk) {
    if (chunk == 0) return kvq8_decode_chunk_tokens(batch, nkv, max_ctx_len);
    if (chunk < 0 || chunk % kChunkUnit != 0 || chunk > 64 * kChunkUnit) return -1;
    return chunk;
}

extern "C" size_t kvq8_decode_workspace_size(int batch, int nq, int nkv, int max_ctx_len, int chunk) {
    if (batch < 0 || nq < 1 || nkv < 1 || max_ctx_len < 0) return 0;
    const int ch = resolve_chunk8(batch, nkv, max_ctx_len, chunk);
    if (ch <= 0) return 0;
    return decode_workspace_bytes(batch, nq, (max_ctx_len + ch - 1) / ch);
}

// Decode without a caller workspace: the chunk partials go to `scratch`, a
// library-owned device array (each device holds its own copy while the
// process runs).  Its device address is looked up once per device, with that
// device current; host code uses only that address, never the array's name.
constexpr size_t kScratchBytes = KVQ8_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (KVQ8_EINVAL when `stream`
// belongs to another device, KVQ8_EHIP when the runtime fails).
int scratch_address(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ8_EHIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return KVQ8_EHIP;
        if (sdev != dev) return KVQ8_EINVAL;
    }
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ8_EHIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return KVQ8_OK;
}
}  // namespace

// kvq8_decode_attn with its workspace, or (own_scratch) with the library's
// scratch array.  Every argument is checked before the scratch address is
// looked up or anything is launched.
static int decode8(float* out, const float* q, int batch, int nq, const int8_t* k_cache, const int8_t* v_cache,
                   const float* k_scale, const float* v_scale, int n_blocks, int kv_bs, int nkv, int hd,
                   const int32_t* block_tables, int max_blocks_per_seq, const int32_t* ctx_lens, int max_ctx_len,
                   float sm_scale, int chunk, void* workspace, size_t workspace_bytes, void* stream,
                   bool own_scratch) {
    if (!decode_shape_ok(batch, nq, nkv, hd, kv_bs) || n_blocks < 1 || max_blocks_per_seq < 1) return KVQ8_ESHAPE;
    if (!rows_fit_u32(n_blocks, kv_bs, nkv)) return KVQ8_ESHAPE;
    if (max_ctx_len < 0 || !score_scale_ok(sm_scale)) return KVQ8_EINVAL;
    const int ch = resolve_chunk8(batch, nkv, max_ctx_len, chunk);
    if (ch <= 0) return KVQ8_ESHAPE;
    if (batch == 0) return KVQ8_OK;
    if (!out || !q || !k_cache || !v_cache || !k_scale || !v_scale || !block_tables || !ctx_lens)
        return KVQ8_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return KVQ8_EINVAL;
    const size_t need = kvq8_decode_workspace_size(batch, nq, nkv, max_ctx_len, chunk);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (own_scratch) {
        if (need > kScratchBytes) return KVQ8_EWORKSPACE;
        const int st = scratch_address(s, &workspace);
        if (st != KVQ8_OK) return st;
    } else if (!workspace || workspace_bytes < need || !aligned16(workspace)) {
        return KVQ8_EWORKSPACE;
    }

    DecodeArgs a = {};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.ks = k_scale;
    a.vs = v_scale;
    a.r8 = Region{block_tables, ctx_lens, max_blocks_per_seq, max_ctx_len, n_blocks, (max_ctx_len + ch - 1) / ch};
    a.r4 = Region{nullptr, nullptr, 1, 0, 0, 0};
    a.nq = nq;
    a.nkv = nkv;
    a.log2_bs = ilog2(kv_bs);
    a.batch = batch;
    a.tiles_per_wave = ch / kChunkUnit;
    a.score_scale = score_scale(sm_scale) * kLog2e;
    bind_workspace(a, workspace);
    return launch_decode(a, out, s);
}

extern "C" int kvq8_decode_attn(float* out, const float* q, int batch, int nq, const int8_t* k_cache,
                                const int8_t* v_cache, const float* k_scale, const float* v_scale, int n_blocks,
                                int kv_bs, int nkv, int hd, const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* ctx_lens, int max_ctx_len, float sm_scale, int chunk,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return decode8(out, q, batch, nq, k_cache, v_cache, k_scale, v_scale, n_blocks, kv_bs, nkv, hd, block_tables,
                   max_blocks_per_seq, ctx_lens, max_ctx_len, sm_scale, chunk, workspace, workspace_bytes, stream,
                   false);
}

extern "C" int kvq8_decode_attn_noalloc(float* out, const float* q, int batch, int nq, const int8_t* k_cache,
                                        const int8_t* v_cache, const float* k_scale, const float* v_scale,
                                        int n_blocks, int kv_bs, int nkv, int hd, const int32_t* block_tables,
                                        int max_blocks_per_seq, const int32_t* ctx_lens, int max_ctx_len,
                                        float sm_scale, int chunk, void* stream) {
    return decode8(out, q, batch, nq, k_cache, v_cache, k_scale, v_scale, n_blocks, kv_bs, nkv, hd, block_tables,
                   max_blocks_per_seq, ctx_lens, max_ctx_len, sm_scale, chunk, nullptr, 0, stream, true);
}

extern "C" int kvq8_append_decode_attn(float* out, const float* q, int batch, int nq, const void* k_new,
                                       const void* v_new, int dtype, int8_t* k_cache, int8_t* v_cache,
                                       float* k_scale, float* v_scale, int n_blocks, int kv_bs, int nkv, int hd,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* ctx_lens, int max_ctx_len, float sm_scale, int chunk,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    if (!decode_shape_ok(batch, nq, nkv, hd, kv_bs) || n_blocks < 1 || max_blocks_per_seq < 1) return KVQ8_ESHAPE;
    if (!rows_fit_u32(n_blocks, kv_bs, nkv)) return KVQ8_ESHAPE;
    if (max_ctx_len < 0 || dtype < KVQ8_F32 || dtype > KVQ8_F16 || !score_scale_ok(sm_scale))
        return KVQ8_EINVAL;
    const int ch = resolve_chunk8(batch, nkv, max_ctx_len, chunk);
    if (ch <= 0) return KVQ8_ESHAPE;
    if (batch == 0) return KVQ8_OK;
    if (!out || !q || !k_new || !v_new || !k_cache || !v_cache || !k_scale || !v_scale || !block_tables ||
        !ctx_lens)
        return KVQ8_EINVAL;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return KVQ8_EINVAL;
    const size_t need = kvq8_decode_workspace_size(batch, nq, nkv, max_ctx_len, chunk);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KVQ8_EWORKSPACE;

    DecodeArgs a = {};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.ks = k_scale;
    a.vs = v_scale;
    a.kc_w = k_cache;
    a.vc_w = v_cache;
    a.ks_w = k_scale;
    a.vs_w = v_scale;
    a.k_new = k_new;
    a.v_new = v_new;
    a.r8 = Region{block_tables, ctx_lens, max_blocks_per_seq, max_ctx_len, n_blocks, (max_ctx_len + ch - 1) / ch};
    a.r4 = Region{nullptr, nullptr, 1, 0, 0, 0};
    a.nq = nq;
    a.nkv = nkv;
    a.log2_bs = ilog2(kv_bs);
    a.batch = batch;
    a.tiles_per_wave = ch / kChunkUnit;
    a.score_scale = score_scale(sm_scale) * kLog2e;
    bind_workspace(a, workspace);
    return launch_decode(a, out, static_cast<hipStream_t>(stream), dtype);
}

extern "C" int kvq8_qk_partials(int32_t* partials, const float* q, int batch, int nq, const int8_t* k_cache,
                                int n_blocks, int kv_bs, int nkv, int hd, const int32_t* block_tables,
                                int max_blocks_per_seq, const int32_t* ctx_lens, int max_ctx_len, void* stream) {
    if (!decode_shape_ok(batch, nq, nkv, hd, kv_bs) || n_blocks < 1 || max_blocks_per_seq < 1) return KVQ8_ESHAPE;
    if (!rows_fit_u32(n_blocks, kv_bs, nkv)) return KVQ8_ESHAPE;
    if (max_ctx_len < 0) return KVQ8_EINVAL;
    if (batch == 0 || max_ctx_len == 0) return KVQ8_OK;
    if (!partials || !q || !k_cache || !block_tables || !ctx_lens) return KVQ8_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache)) return KVQ8_EINVAL;
    DecodeArgs a = {};
    a.q = q;
    a.kc = k_cache;
    a.r8 = Region{block_tables, ctx_lens, max_blocks_per_seq, max_ctx_len, n_blocks, 1};
    a.nq = nq;
    a.nkv = nkv;
    a.log2_bs = ilog2(kv_bs);
    a.batch = batch;
    const int n_groups = (max_ctx_len + kChunkUnit - 1) / kChunkUnit;
    if ((long)batch * nkv * n_groups > 0x7FFFFFFFL) return KVQ8_ESHAPE;
    const dim3 grid(batch * nkv * n_groups), block(kWGThreads);
    if (kv_bs < 16)
        return launch(kvq8_qk_partials_kernel<true>, grid, block, static_cast<hipStream_t>(stream), a, partials,
                      n_groups);
    return launch(kvq8_qk_partials_kernel<false>, grid, block, static_cast<hipStream_t>(stream), a, partials,
                  n_groups);
}

extern "C" int kvq4_decode_chunk_tokens(int batch, int nkv, int max_len4, int max_len8) {
    if (batch < 0 || nkv < 1 || max_len4 < 0 || max_len8 < 0) return 0;
    // two workgroups per CU: at least 512 of them; few (sequence, head) units
    // are long enough to take 8 tiles per wave, many balance better with 4
    const long units = (long)batch * nkv;
    return default_tiles_per_wave(units, (long)max_len4 + max_len8, units <= 16 ? 8 : 4, 512) * kChunkUnit;
}

static int resolve_chunk4(int batch, int nkv, int max_len4, int max_len8, int chunk) {
    if (chunk == 0) return kvq4_decode_chunk_tokens(batch, nkv, max_len4, max_len8);
    if (chunk < 0 || chunk % kChunkUnit != 0 || chunk > 64 * kChunkUnit) return -1;
    return chunk;
}

extern "C" size_t kvq4_decode_workspace_size(int batch, int nq, int nkv, int max_len4, int max_len8, int chunk) {
    if (batch < 0 || nq < 1 || nkv < 1 || max_len4 < 0 || max_len8 < 0) return 0;
    const int ch = resolve_chunk4(batch, nkv, max_len4, max_len8, chunk);
    if (ch <= 0) return 0;
    return decode_workspace_bytes(batch, nq, (max_len4 + ch - 1) / ch + (max_len8 + ch - 1) / ch);
}

extern "C" int kvq4_decode_attn(float* out, const float* q, int batch, int nq, const uint8_t* k_cache4,
                                const uint8_t* v_cache4, const uint16_t* k_scale4, const uint16_t* k_zero4,
                                const uint16_t* v_scale4, const uint16_t* v_zero4, int n_blocks4,
                                const int32_t* block_tables4, int max_blocks_per_seq4, const int32_t* lens4,
                                int max_len4, const int8_t* k_cache8, const int8_t* v_cache8,
                                const float* k_scale8, const float* v_scale8, int n_blocks8,
                                const int32_t* block_tables8, int max_blocks_per_seq8, const int32_t* lens8,
                                int max_len8, int kv_bs, int nkv, int hd, float sm_scale, int chunk,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (!decode_shape_ok(batch, nq, nkv, hd, kv_bs)) return KVQ8_ESHAPE;
    if (n_blocks4 < 1 || n_blocks8 < 1 || max_blocks_per_seq4 < 1 || max_blocks_per_seq8 < 1) return KVQ8_ESHAPE;
    if (max_len4 < 0 || max_len8 < 0 || !score_scale_ok(sm_scale)) return KVQ8_EINVAL;
    const int ch = resolve_chunk4(batch, nkv, max_len4, max_len8, chunk);
    if (ch <= 0) return KVQ8_ESHAPE;
    if (batch == 0) return KVQ8_OK;
    if (!out || !q || !k_cache4 || !v_cache4 || !k_scale4 || !k_zero4 || !v_scale4 || !v_zero4 ||
        !block_tables4 || !lens4 || !k_cache8 || !v_cache8 || !k_scale8 || !v_scale8 || !block_tables8 || !lens8)
        return KVQ8_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache4) || !aligned16(v_cache4) || !aligned16(k_cache8) ||
        !aligned16(v_cache8))
        return KVQ8_EINVAL;
    // both groups' binary16 scale (zero point) of a row are read as one word
    if (((uintptr_t)k_scale4 | (uintptr_t)k_zero4 | (uintptr_t)v_scale4 | (uintptr_t)v_zero4) & 3u) return KVQ8_EINVAL;
    if (!rows_fit_u32(n_blocks4, kv_bs, nkv) || !rows_fit_u32(n_blocks8, kv_bs, nkv)) return KVQ8_ESHAPE;
    const size_t need = kvq4_decode_workspace_size(batch, nq, nkv, max_len4, max_len8, chunk);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KVQ8_EWORKSPACE;

    DecodeArgs a = {};
    a.q = q;
    a.kc = k_cache8;
    a.vc = v_cache8;
    a.ks = k_scale8;
    a.vs = v_scale8;
    a.k4 = k_cache4;
    a.v4 = v_cache4;
    a.k4s = k_scale4;
    a.k4z = k_zero4;
    a.v4s = v_scale4;
    a.v4z = v_zero4;
    a.r8 = Region{block_tables8, lens8, max_blocks_per_seq8, max_len8, n_blocks8, (max_len8 + ch - 1) / ch};
    a.r4 = Region{block_tables4, lens4, max_blocks_per_seq4, max_len4, n_blocks4, (max_len4 + ch - 1) / ch};
    a.nq = nq;
    a.nkv = nkv;
    a.log2_bs = ilog2(kv_bs);
    a.batch = batch;
    a.tiles_per_wave = ch / kChunkUnit;
    a.score_scale = score_scale(sm_scale) * kLog2e;
    bind_workspace(a, workspace);
    return launch_decode(a, out, static_cast<hipStream_t>(stream));
}

// ----------------------------------------------------------------------------
// banded group cache: 2-bit, int4 and int8 bands ([P4] Sec. 3.3)
// ----------------------------------------------------------------------------

extern "C" int kvq2_decode_chunk_tokens(int batch, int nkv, int max_len2, int max_len4, int max_len8) {
    if (batch < 0 || nkv < 1 || max_len2 < 0 || max_len4 < 0 || max_len8 < 0) return 0;
    const long units = (long)batch * nkv;
    return default_tiles_per_wave(units, (long)max_len2 + max_len4 + max_len8, units <= 16 ? 8 : 4, 512) *
           kChunkUnit;
}

static int resolve_chunk2(int batch, int nkv, int max_len2, int max_len4, int max_len8, int chunk) {
    if (chunk == 0) return kvq2_decode_chunk_tokens(batch, nkv, max_len2, max_len4, max_len8);
    if (chunk < 0 || chunk % kChunkUnit != 0 || chunk > 64 * kChunkUnit) return -1;
    return chunk;
}

extern "C" size_t kvq2_decode_workspace_size(int batch, int nq, int nkv, int max_len2, int max_len4, int max_len8,
                                             int chunk) {
    if (batch < 0 || nq < 1 || nkv < 1 || max_len2 < 0 || max_len4 < 0 || max_len8 < 0) return 0;
    const int ch = resolve_chunk2(batch, nkv, max_len2, max_len4, max_len8, chunk);
    if (ch <= 0) return 0;
    return decode_workspace_bytes(batch, nq,
                                  (max_len2 + ch - 1) / ch + (max_len4 + ch - 1) / ch + (max_len8 + ch - 1) / ch);
}

extern "C" int kvq2_decode_attn(float* out, const float* q, int batch, int nq, const uint8_t* k_cache2,
                                const uint8_t* v_cache2, const uint16_t* k_scale2, const uint16_t* k_zero2,
                                const uint16_t* v_scale2, const uint16_t* v_zero2, int n_blocks2,
                                const int32_t* block_tables2, int max_blocks_per_seq2, const int32_t* lens2,
                                int max_len2, const uint8_t* k_cache4, const uint8_t* v_cache4,
                                const uint16_t* k_scale4, const uint16_t* k_zero4, const uint16_t* v_scale4,
                                const uint16_t* v_zero4, int n_blocks4, const int32_t* block_tables4,
                                int max_blocks_per_seq4, const int32_t* lens4, int max_len4, const int8_t* k_cache8,
                                const int8_t* v_cache8, const float* k_scale8, const float* v_scale8, int n_blocks8,
                                const int32_t* block_tables8, int max_blocks_per_seq8, const int32_t* lens8,
                                int max_len8, int kv_bs, int nkv, int hd, float sm_scale, int chunk,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (!decode_shape_ok(batch, nq, nkv, hd, kv_bs)) return KVQ8_ESHAPE;
    if (n_blocks2 < 1 || n_blocks4 < 1 || n_blocks8 < 1 || max_blocks_per_seq2 < 1 || max_blocks_per_seq4 < 1 ||
        max_blocks_per_seq8 < 1)
        return KVQ8_ESHAPE;
    if (max_len2 < 0 || max_len4 < 0 || max_len8 < 0 || !score_scale_ok(sm_scale)) return KVQ8_EINVAL;
    const int ch = resolve_chunk2(batch, nkv, max_len2, max_len4, max_len8, chunk);
    if (ch <= 0) return KVQ8_ESHAPE;
    if (batch == 0) return KVQ8_OK;
    if (!out || !q || !k_cache2 || !v_cache2 || !k_scale2 || !k_zero2 || !v_scale2 || !v_zero2 || !block_tables2 ||
        !lens2 || !k_cache4 || !v_cache4 || !k_scale4 || !k_zero4 || !v_scale4 || !v_zero4 || !block_tables4 ||
        !lens4 || !k_cache8 || !v_cache8 || !k_scale8 || !v_scale8 || !block_tables8 || !lens8)
        return KVQ8_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache2) || !aligned16(v_cache2) || !aligned16(k_cache4) ||
        !aligned16(v_cache4) || !aligned16(k_cache8) || !aligned16(v_cache8))
        return KVQ8_EINVAL;
    // both groups' binary16 scale (zero point) of a row are read as one word
    if (((uintptr_t)k_scale2 | (uintptr_t)k_zero2 | (uintptr_t)v_scale2 | (uintptr_t)v_zero2 | (uintptr_t)k_scale4 |
         (uintptr_t)k_zero4 | (uintptr_t)v_scale4 | (uintptr_t)v_zero4) & 3u)
        return KVQ8_EINVAL;
    if (!rows_fit_u32(n_blocks2, kv_bs, nkv) || !rows_fit_u32(n_blocks4, kv_bs, nkv) ||
        !rows_fit_u32(n_blocks8, kv_bs, nkv))
        return KVQ8_ESHAPE;
    const size_t need = kvq2_decode_workspace_size(batch, nq, nkv, max_len2, max_len4, max_len8, chunk);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KVQ8_EWORKSPACE;

    BandArgs a = {};
    a.q = q;
    a.kc = k_cache8;
    a.vc = v_cache8;
    a.ks = k_scale8;
    a.vs = v_scale8;
    a.k4 = k_cache4;
    a.v4 = v_cache4;
    a.k4s = k_scale4;
    a.k4z = k_zero4;
    a.v4s = v_scale4;
    a.v4z = v_zero4;
    a.k2 = k_cache2;
    a.v2 = v_cache2;
    a.k2s = k_scale2;
    a.k2z = k_zero2;
    a.v2s = v_scale2;
    a.v2z = v_zero2;
    a.r8 = Region{block_tables8, lens8, max_blocks_per_seq8, max_len8, n_blocks8, (max_len8 + ch - 1) / ch};
    a.r4 = Region{block_tables4, lens4, max_blocks_per_seq4, max_len4, n_blocks4, (max_len4 + ch - 1) / ch};
    a.r2 = Region{block_tables2, lens2, max_blocks_per_seq2, max_len2, n_blocks2, (max_len2 + ch - 1) / ch};
    a.nq = nq;
    a.nkv = nkv;
    a.log2_bs = ilog2(kv_bs);
    a.batch = batch;
    a.tiles_per_wave = ch / kChunkUnit;
    a.score_scale = score_scale(sm_scale) * kLog2e;
    bind_workspace(a, workspace);
    return launch_decode(a, out, static_cast<hipStream_t>(stream));
}
