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

// Quantize a 128-value row held by an aligned 8-lane group, 16 values per
// lane: the lane's 16 codes (packed) and the row's step d = amax / 127.
//
// The code is roundf(x / d) clamped to +-127.  f = fma(x, rcp(d), 384.5 +
// 2^-13) lies in [256, 512) (|x / d| <= 127), so its unit is 2^-15 and its
// mantissa is (x * rcp(d) + 128.5) * 2^15, rounded, plus 4: bits 15..22 are
// 128 + the code and bits 0..14 the fraction plus 4.  Where those low bits
// are 0..7 the quotient lies within 2^-12 of a half-integer and the lane
// divides instead (about 0.02% of the values); elsewhere it lies at least
// 3.5 * 2^-15 from one, more than one rcp error (127 * 2^-23 < 2^-16) plus
// the division's rounding, so the floor read from f is roundf of the
// correctly rounded quotient.  Four code bytes are gathered by a rotation
// each and two byte permutes; the xor turns 128 + c into c's two's complement.
__device__ __forceinline__ void quantize_row8x16(const float (&x)[16], uint4& codes, float& d) {
#pragma clang fp contract(off)
    constexpr float kMagic = 384.5001220703125f;     // 256 + 128.5 + 2^-13
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
    amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
    amax = fmaxf(amax, dpp_f<kDppHalfMirror>(amax));
    if (amax < 1e-6f) amax = 1.0f;
    d = amax / 127.0f;
    const float rd = __builtin_amdgcn_rcpf(d);
    uint32_t f[16];
    uint64_t slow[16];                               // wave masks of the lanes that divide
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        f[e] = __float_as_uint(__builtin_fmaf(x[e], rd, kMagic));
        slow[e] = __builtin_amdgcn_ballot_w64((f[e] & 0x7FF8u) == 0u);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (slow[e] != 0) {                         // rare: one wave-uniform test per value
            const float r = fminf(fmaxf(roundf(x[e] / d), -127.0f), 127.0f);
            f[e] = ((slow[e] >> (threadIdx.x & 63)) & 1) ? (uint32_t)((int)r + 128) << 15 : f[e];
        }
    }
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        uint32_t t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = __builtin_amdgcn_alignbit(f[4 * h + i], f[4 * h + i], 15u);
        w[h] = (__builtin_amdgcn_perm(t[1], t[0], 0x0C0C0400u) | __builtin_amdgcn_perm(t[3], t[2], 0x04000C0Cu)) ^
               0x80808080u;
    }
    codes = make_uint4(w[0], w[1], w[2], w[3]);
}

// Row numbers of the pool (slot * nkv + head) fit in 32 bits: the host
// checks n_slots * nkv, and ns_cap = min(n_slots, 2^31) turns the slot test
// into one unsigned compare.
// 16 code bytes of a lane as a native vector (the operand type of the
// non-temporal store builtin)
typedef uint32_t Codes16 __attribute__((ext_vector_type(4)));

template <int DT>
__global__ __launch_bounds__(256) void kvq8_quantize_append_kernel(
    int8_t* __restrict__ kc, int8_t* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs,
    uint32_t ns_cap, DivN nkv, const void* __restrict__ k_new, const void* __restrict__ v_new,
    int n_rows, const int32_t* __restrict__ slots) {
    const int l8 = threadIdx.x & 7;
    const int kind = (threadIdx.x >> 3) & 1;       // rows alternate K, V (k * 32 is even)
    const int p = q8_rot_group(nkv.n);
    float x[kRowsPerGroup][16];
    int trs[kRowsPerGroup];
    uint32_t slot[kRowsPerGroup];
    // rows past the end load the last row again and store nothing; indices
    // fit in 32 bits (the host checks the row count)
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        const int row = (int)blockIdx.x * kRowsPerBlock + k * 32 + (threadIdx.x >> 3);
        const int tr = min(row, n_rows - 1) >> 1;  // token * nkv + kv-head
        trs[k] = tr;
        load_new16<DT>(kind ? v_new : k_new, (size_t)tr * kHD + 16 * l8, x[k]);
        slot[k] = (uint32_t)slots[div_n(tr, nkv)];
    }
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        uint4 codes;
        float d;
        quantize_row8x16(x[k], codes, d);         // every lane of the row takes part (DPP)
        const int row = (int)blockIdx.x * kRowsPerBlock + k * 32 + (threadIdx.x >> 3);
        if (row >= n_rows || slot[k] >= ns_cap) continue;   // uniform per 8-lane row
        const int kh = trs[k] - div_n(trs[k], nkv) * nkv.n;
        const uint32_t base = slot[k] * (uint32_t)nkv.n;
        // streaming store: measured on MI355X, the 64K-token write took 63 us
        // this way against 80 us with the default policy (the bf16 inputs
        // loaded the same way were no faster)
        __builtin_nontemporal_store(Codes16{codes.x, codes.y, codes.z, codes.w},
                                    reinterpret_cast<Codes16*>((kind ? vc : kc) +
                                                               (size_t)(base + (uint32_t)q8_col(kh, slot[k], p)) * kHD +
                                                               16 * l8));
        if (l8 == 0) (kind ? vs : ks)[base + (uint32_t)kh] = d;
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
    // pool rows (slot * nkv + head) are 32-bit in the kernel: 2^32 rows would
    // take 512 GiB of codes
    if (n_slots * nkv > 0xFFFFFFFFL) return KVQ8_ESHAPE;
    const dim3 grid((unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int st;
    switch (dtype) {
        case KVQ8_F32:
            st = launch(kvq8_quantize_append_kernel<KVQ8_F32>, grid, block, s, k_cache, v_cache, k_scale,
                               v_scale, slot_cap(n_slots), make_divn(nkv), k_new, v_new, (int)n_rows, slots);
            break;
        case KVQ8_BF16:
            st = launch(kvq8_quantize_append_kernel<KVQ8_BF16>, grid, block, s, k_cache, v_cache, k_scale,
                               v_scale, slot_cap(n_slots), make_divn(nkv), k_new, v_new, (int)n_rows, slots);
            break;
        default:
            st = launch(kvq8_quantize_append_kernel<KVQ8_F16>, grid, block, s, k_cache, v_cache, k_scale,
                               v_scale, slot_cap(n_slots), make_divn(nkv), k_new, v_new, (int)n_rows, slots);
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
