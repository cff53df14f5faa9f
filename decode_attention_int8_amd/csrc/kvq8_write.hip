// Write path of the int8 KV cache and the query-quantization export.
//
// kvq8_quantize_append_kernel: one (token, kv-head, K-or-V) row of 128 values
// per 16 consecutive lanes, 8 values per lane; each 16-lane group handles 4
// rows, so a 256-thread workgroup quantizes 64 rows.  Each lane reads 32 B (float32) or 16 B (bf16 / f16) of
// its row and writes 8 B of codes: fully coalesced 128-B row stores into the
// paged cache ([P2] Sec. 2 write path; rule of [P1] Sec. 2).
#include "kvq8.h"
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

template <int DT>
__device__ __forceinline__ void load8(const void* base, size_t elem_off, float (&x)[8]) {
    if constexpr (DT == KVQ8_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
        float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem_off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == KVQ8_BF16) {
                x[2 * i] = __uint_as_float(w[i] << 16);
                x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            } else {
                x[2 * i] = half_bits_f(w[i] & 0xFFFFu);
                x[2 * i + 1] = half_bits_f(w[i] >> 16);
            }
        }
    }
}

// Rows per 16-lane group: all of a group's loads go out before it quantizes,
// so each wave keeps kRowsPerGroup x 4 rows in flight.
constexpr int kRowsPerGroup = 4;
constexpr int kRowsPerBlock = 16 * kRowsPerGroup;

template <int DT>
__global__ __launch_bounds__(256) void kvq8_quantize_append_kernel(
    int8_t* __restrict__ kc, int8_t* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs,
    long n_slots, int nkv, const void* __restrict__ k_new, const void* __restrict__ v_new,
    long n_rows, const int32_t* __restrict__ slots) {
    const int l16 = threadIdx.x & 15;
    float x[kRowsPerGroup][8];
    long slot[kRowsPerGroup];
    // rows past the end load the last row again and store nothing
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        const long row = min((long)blockIdx.x * kRowsPerBlock + k * 16 + (threadIdx.x >> 4), n_rows - 1);
        const int kind = (int)(row & 1);           // 0 = K, 1 = V
        const long tr = row >> 1;                  // token * nkv + kv-head
        load8<DT>(kind ? v_new : k_new, (size_t)tr * kHD + 8 * l16, x[k]);
        slot[k] = slots[tr / nkv];
    }
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        const long row = (long)blockIdx.x * kRowsPerBlock + k * 16 + (threadIdx.x >> 4);
        uint32_t lo, hi;
        float d;
        quantize_row16x8(x[k], lo, hi, d);         // every lane of the row takes part (DPP)
        if (row >= n_rows || slot[k] < 0 || slot[k] >= n_slots) continue;   // uniform per 16-lane row
        const int kind = (int)(row & 1);
        const long tr = row >> 1;
        const long tok = tr / nkv;
        const size_t dst = (size_t)slot[k] * nkv + (size_t)(tr - tok * nkv);
        *reinterpret_cast<uint2*>((kind ? vc : kc) + dst * kHD + 8 * l16) = make_uint2(lo, hi);
        if (l16 == 0) (kind ? vs : ks)[dst] = d;
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
    const long n_slots = (long)n_blocks * kv_bs;
    const dim3 grid((unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (dtype) {
        case KVQ8_F32:
            hipLaunchKernelGGL(kvq8_quantize_append_kernel<KVQ8_F32>, grid, block, 0, s, k_cache, v_cache, k_scale,
                               v_scale, n_slots, nkv, k_new, v_new, n_rows, slots);
            break;
        case KVQ8_BF16:
            hipLaunchKernelGGL(kvq8_quantize_append_kernel<KVQ8_BF16>, grid, block, 0, s, k_cache, v_cache, k_scale,
                               v_scale, n_slots, nkv, k_new, v_new, n_rows, slots);
            break;
        default:
            hipLaunchKernelGGL(kvq8_quantize_append_kernel<KVQ8_F16>, grid, block, 0, s, k_cache, v_cache, k_scale,
                               v_scale, n_slots, nkv, k_new, v_new, n_rows, slots);
            break;
    }
    return launch_status();
}

extern "C" int kvq8_quantize_q(int8_t* qi, float* qsc, const float* q, int n_vectors, int hd, void* stream) {
    if (hd != kHD) return KVQ8_ESHAPE;
    if (n_vectors < 0) return KVQ8_EINVAL;
    if (n_vectors == 0) return KVQ8_OK;
    if (!qi || !qsc || !q || !aligned16(q) || !aligned16(qi)) return KVQ8_EINVAL;
    const dim3 grid((unsigned)((n_vectors + kMaxRows - 1) / kMaxRows)), block(256);
    hipLaunchKernelGGL(kvq8_quantize_q_kernel, grid, block, 0, static_cast<hipStream_t>(stream), qi, qsc, q,
                       (long)n_vectors);
    return launch_status();
}
