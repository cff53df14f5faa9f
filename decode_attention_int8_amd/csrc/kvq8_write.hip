// Write path of the int8 KV cache and the query-quantization export.
//
// kvq8_quantize_append_kernel: one (token, kv-head, K-or-V) row of 128 values
// per 8 consecutive lanes, 16 values per lane; each 8-lane group handles 2
// rows, so a 256-thread workgroup quantizes 64 rows.  Each lane reads 64 B
// (float32) or 32 B (bf16 / f16) of its row and writes 16 B of codes: whole
// 128-B rows per 8 lanes ([P2] Sec. 2 write path; rule of [P1] Sec. 2, the
// same quantizer as the decode's fused write path).
#include "kvq8.h"
#include "kvq_device.h"
#include "kvq_host.h"
#include "kvq_decode_core.h"

namespace kvq {

// Rows per 8-lane group: both rows' loads go out before either is quantized.
constexpr int kRowsPerGroup = 2;
constexpr int kRowsPerBlock = 32 * kRowsPerGroup;

template <int DT>
__global__ __launch_bounds__(256) void kvq8_quantize_append_kernel(
    int8_t* __restrict__ kc, int8_t* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs,
    long n_slots, DivN nkv, const void* __restrict__ k_new, const void* __restrict__ v_new,
    int n_rows, const int32_t* __restrict__ slots) {
    const int l8 = threadIdx.x & 7;
    const int p = q8_rot_group(nkv.n);
    float x[kRowsPerGroup][16];
    long dst[kRowsPerGroup];     // destination row (slot * nkv + head), -1 to skip
    long cdst[kRowsPerGroup];    // its code row (slot * nkv + column)
    // rows past the end load the last row again and store nothing; indices
    // fit in 32 bits (the host checks the row count)
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        const int row = (int)blockIdx.x * kRowsPerBlock + k * 32 + (threadIdx.x >> 3);
        const int rc = min(row, n_rows - 1);
        const int tr = rc >> 1;                    // token * nkv + kv-head
        const int tok = div_n(tr, nkv);
        load_new16<DT>((rc & 1) ? v_new : k_new, (size_t)tr * kHD + 16 * l8, x[k]);
        const long slot = slots[tok];
        const int kh = tr - tok * nkv.n;
        dst[k] = (row < n_rows && slot >= 0 && slot < n_slots) ? slot * nkv.n + kh : -1;
        cdst[k] = slot * nkv.n + q8_col(kh, slot, p);
    }
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        uint4 codes;
        float d;
        quantize_row8x16(x[k], codes, d);         // every lane of the row takes part (DPP)
        if (dst[k] < 0) continue;                  // uniform per 8-lane row
        const int kind = (threadIdx.x >> 3) & 1;   // rows alternate K, V (k * 32 is even)
        *reinterpret_cast<uint4*>((kind ? vc : kc) + (size_t)cdst[k] * kHD + 16 * l8) = codes;
        if (l8 == 0) (kind ? vs : ks)[dst[k]] = d;
    }
}

// One 8-lane group per query vector; lane j quantizes values 16j .. 16j+15.
// The decode kernels' query quantization, exported: a workgroup of 256
// threads quantizes 8 rows into LDS and copies codes and scales out.
__global__ __launch_bounds__(256) void kvq8_quantize_q_kernel(int8_t* __restrict__ qi, float* __restrict__ qsc,
                                                              const float* __restrict__ q, long n_vectors) {
    __shared__ QSmem sm;
    const long row0 = (long)blockIdx.x * kMaxRows;
    const int n = (int)min((long)kMaxRows, n_vectors - row0);
    const float4 x = load_q4(q + (size_t)row0 * kHD, n);
    quantize_q4(x, n, sm);
    lds_barrier();
    const int t = threadIdx.x;
    if ((t >> 5) < n) {
        reinterpret_cast<uint32_t*>(qi + (size_t)row0 * kHD)[t] = sm.qc[t >> 5][t & 31];
        if ((t & 31) < kHD / kQBlock) qsc[(size_t)row0 * (kHD / kQBlock) + 4 * (t >> 5) + (t & 31)] =
            sm.qs[t >> 5][t & 31];
    }
}

}  // namespace kvq

using namespace kvq;

extern "C" int kvq8_quantize_append(int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                                    int n_blocks, int kv_bs, int nkv, int hd,
                                    const void* k_new, const void* v_new, int dtype, int n_tokens,
                                    const int32_t* slots, void* stream) {
    if (hd != kHD || !valid_block_size(kv_bs) || nkv < 1 || n_blocks < 1) return KVQ8_ESHAPE;
    if (n_tokens < 0 || dtype < KVQ8_F32 || dtype > KVQ8_F16) return KVQ8_EINVAL;
    if (n_tokens == 0) return KVQ8_OK;
    if (!k_cache || !v_cache || !k_scale || !v_scale || !k_new || !v_new || !slots) return KVQ8_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)) return KVQ8_EINVAL;
    const long n_rows = (long)n_tokens * nkv * 2;
    if (n_rows > 0x7FFFFFFFL - kRowsPerBlock) return KVQ8_ESHAPE;
    const long n_slots = (long)n_blocks * kv_bs;
    const dim3 grid((unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int st;
    switch (dtype) {
        case KVQ8_F32:
            st = launch(kvq8_quantize_append_kernel<KVQ8_F32>, grid, block, s, k_cache, v_cache, k_scale,
                               v_scale, n_slots, make_divn(nkv), k_new, v_new, (int)n_rows, slots);
            break;
        case KVQ8_BF16:
            st = launch(kvq8_quantize_append_kernel<KVQ8_BF16>, grid, block, s, k_cache, v_cache, k_scale,
                               v_scale, n_slots, make_divn(nkv), k_new, v_new, (int)n_rows, slots);
            break;
        default:
            st = launch(kvq8_quantize_append_kernel<KVQ8_F16>, grid, block, s, k_cache, v_cache, k_scale,
                               v_scale, n_slots, make_divn(nkv), k_new, v_new, (int)n_rows, slots);
            break;
    }
    return st;
}

extern "C" int kvq8_quantize_q(int8_t* qi, float* qsc, const float* q, int n_vectors, int hd, void* stream) {
    if (hd != kHD) return KVQ8_ESHAPE;
    if (n_vectors < 0) return KVQ8_EINVAL;
    if (n_vectors == 0) return KVQ8_OK;
    if (!qi || !qsc || !q || !aligned16(q) || !aligned16(qi)) return KVQ8_EINVAL;
    const dim3 grid((unsigned)((n_vectors + kMaxRows - 1) / kMaxRows)), block(256);
    return launch(kvq8_quantize_q_kernel, grid, block, static_cast<hipStream_t>(stream), qi, qsc, q,
                  (long)n_vectors);
}
