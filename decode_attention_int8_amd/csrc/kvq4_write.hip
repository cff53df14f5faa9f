// Write path of the int4 group variant ([P4] Sec. 3.2 quantizer with the
// Sec. 5.2 checklist).
//
// kvq4_quantize_append_kernel: one (token, kv-head, K-or-V) row per 8 lanes,
// 16 values per lane, 4 rows per 8-lane group (loads first); each 64-value
// group is one quad, so its max / min need two quad DPP steps.
// kvq4_requantize_q8_kernel: one row per 16 lanes, 8 values per lane (each
// group an aligned 8-lane half row).
#include "kvq8.h"
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

template <int DT>
__device__ __forceinline__ void load8_any(const void* base, size_t elem_off, float (&x)[8]) {
    if constexpr (DT == KVQ8_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
        const float4 u = p[0], v = p[1];
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
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

__device__ __forceinline__ uint16_t f16_bits_rne(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Quantize the lane's 8 values of a 64-value group held by an aligned 8-lane
// half row: returns 4 packed bytes (value 2k in the high nibble of byte k),
// the binary16 scale and the zero point.
__device__ __forceinline__ void quantize_group8x8(const float (&x)[8], uint32_t& packed, uint16_t& s16,
                                                  uint16_t& z16) {
#pragma clang fp contract(off)
    float mx = x[0], mn = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
        mx = fmaxf(mx, x[e]);
        mn = fminf(mn, x[e]);
    }
    mx = fmaxf(mx, dpp_f<kDppXor1>(mx));
    mn = fminf(mn, dpp_f<kDppXor1>(mn));
    mx = fmaxf(mx, dpp_f<kDppXor2>(mx));
    mn = fminf(mn, dpp_f<kDppXor2>(mn));
    mx = fmaxf(mx, dpp_f<kDppHalfMirror>(mx));
    mn = fminf(mn, dpp_f<kDppHalfMirror>(mn));
    float s32 = (mx == mn) ? 1.0f : (mx - mn) / 15.0f;
    s32 = fmaxf(s32, 1e-7f);
    s16 = f16_bits_rne(s32);
    const float s = half_bits_f(s16);
    // integer zero point in [0, 15]; + 0.0f stores a zero as +0.0
    const float z = fminf(fmaxf(rintf(-mn / s), 0.0f), 15.0f) + 0.0f;
    z16 = f16_bits_rne(z);
    const float rs = __builtin_amdgcn_rcpf(s);
    // code = clamp(rint(x / s + z), 0, 15) with z an integer, the quotient
    // computed only near a half-integer.  Elsewhere the clamped q + z plus
    // 1.5 * 2^23 holds rint(q + z) in its low byte (the addition rounds half
    // to even like rint), so the codes are gathered with byte permutes.
    constexpr float kMagic = 12582912.0f;
    uint32_t cb[8];
    bool slow[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float q = x[e] * rs;
        slow[e] = near_half(q);
        cb[e] = __float_as_uint(__builtin_amdgcn_fmed3f(q + z, 0.0f, 15.0f) + kMagic);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (__builtin_amdgcn_ballot_w64(slow[e]) != 0) {      // rare: one wave-uniform test per value
            const float cd = fminf(fmaxf(rintf(x[e] / s + z), 0.0f), 15.0f);
            cb[e] = slow[e] ? (uint32_t)(int)cd : cb[e];
        }
    }
    // bytes [c0, c1, c2, c3] and [c4 .. c7]; (b << 4) | (b >> 8) puts the
    // pairs (c0, c1) and (c2, c3) in bytes 0 and 2, even element high
    uint32_t pr[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t b = __builtin_amdgcn_perm(cb[4 * h + 1], cb[4 * h], 0x0C0C0400u) |
                           __builtin_amdgcn_perm(cb[4 * h + 3], cb[4 * h + 2], 0x04000C0Cu);
        pr[h] = (b << 4) | (b >> 8);
    }
    packed = __builtin_amdgcn_perm(pr[1], pr[0], 0x06040200u);
}

constexpr int kRowsPerGroup = 4;            // rows per 8-lane group, loads first
constexpr int kRowsPerBlock = 32 * kRowsPerGroup;

// A row's lanes: lane l of the 8-lane group holds elements 64g + 16c ..
// 64g + 16c + 15 with g = l / 4 and c = l % 4 for g = 0, 3 - l % 4 for
// g = 1, so lanes l and 7 - l (one half-mirror DPP step) hold the same c of
// the two groups.  Key rows: the lane's pairs 64g + 16c + 2j go to bytes
// 16c + 8g + j, 8 contiguous bytes.  Value rows: the pair 64g + 4m + 2k, +1
// goes to byte 4m + 2g + k, so words m = 4c .. 4c + 3 take two bytes from
// each lane of the mirror pair; the g = 0 lane writes words 4c, 4c + 1, its
// partner words 4c + 2, 4c + 3.  Row numbers of the pool (slot * nkv + head)
// fit in 32 bits (the host checks n_slots * nkv; ns_cap = min(n_slots,
// 2^31)).
template <int DT>
__global__ __launch_bounds__(256) void kvq4_quantize_append_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, uint16_t* __restrict__ ks, uint16_t* __restrict__ kz,
    uint16_t* __restrict__ vs, uint16_t* __restrict__ vz, uint32_t ns_cap, DivN nkv,
    const void* __restrict__ k_new, const void* __restrict__ v_new, int n_rows, const int32_t* __restrict__ slots) {
    constexpr int kInBytes = DT == KVQ8_F32 ? 4 : 2;
    const int l8 = threadIdx.x & 7;
    const int g = l8 >> 2;
    const int c = g ? 3 - (l8 & 3) : (l8 & 3);
    const int kind = (threadIdx.x >> 3) & 1;       // rows alternate K, V (k * 32 is even)
    const void* src = kind ? v_new : k_new;
    const uint32_t in_off = (uint32_t)(64 * g + 16 * c) * kInBytes;
    const uint32_t out_off = 16u * (uint32_t)c + 8u * (uint32_t)g;   // key and value rows alike
    uint8_t* codes = kind ? vc : kc;
    uint16_t* scales = kind ? vs : ks;
    uint16_t* zeros = kind ? vz : kz;
    Raw16<DT> raw[kRowsPerGroup];
    int trs[kRowsPerGroup];
    uint32_t slot[kRowsPerGroup];
    // rows past the end load the last row again and store nothing; indices
    // fit in 32 bits (the host checks the row count)
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        const int row = (int)blockIdx.x * kRowsPerBlock + k * 32 + (threadIdx.x >> 3);
        const int tr = min(row, n_rows - 1) >> 1;  // token * nkv + kv-head
        trs[k] = tr;
        load_raw16<DT>(src, (size_t)tr * (kHD * kInBytes) + in_off, raw[k]);
        slot[k] = (uint32_t)slots[div_n(tr, nkv)];
    }
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        float x[16];
        unpack_raw16<DT>(raw[k], x);
        uint32_t cb[4], pk[2];
        uint16_t s16, z16;
        quad_group_codes<15>(x, cb, s16, z16);      // every lane of the group takes part (DPP)
        // (b << 4) | (b >> 8) puts the pairs (c0, c1) and (c2, c3) of a code
        // word in bytes 0 and 2, even element high
#pragma unroll
        for (int h = 0; h < 4; ++h) cb[h] = (cb[h] << 4) | (cb[h] >> 8);
        pk[0] = __builtin_amdgcn_perm(cb[1], cb[0], 0x06040200u);   // pairs 0..3: value 2k high in byte k
        pk[1] = __builtin_amdgcn_perm(cb[3], cb[2], 0x06040200u);   // pairs 4..7
        uint2 word;
        if (kind == 0) {
            word = make_uint2(pk[0], pk[1]);
        } else {
            // the g = 0 lane needs the partner's bytes 0..3, the g = 1 lane
            // the partner's bytes 4..7
            const uint32_t r = (uint32_t)dpp_i<kDppHalfMirror>((int)(g ? pk[0] : pk[1]));
            const uint32_t lo = g ? r : pk[0], hi = g ? pk[1] : r;
            word = make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05040100u), __builtin_amdgcn_perm(hi, lo, 0x07060302u));
        }
        const int row = (int)blockIdx.x * kRowsPerBlock + k * 32 + (threadIdx.x >> 3);
        if (row >= n_rows || slot[k] >= ns_cap) continue;   // uniform per 8-lane row
        const uint32_t drow = slot[k] * (uint32_t)nkv.n + (uint32_t)(trs[k] - div_n(trs[k], nkv) * nkv.n);
        *reinterpret_cast<uint2*>(codes + (size_t)drow * (kHD / 2) + out_off) = word;
        if (c == 0) {
            scales[(size_t)drow * 2 + g] = s16;
            zeros[(size_t)drow * 2 + g] = z16;
        }
    }
}

// Store one row: lane l16 packed the pairs of its 8 values (elements 8 l16 ..
// 8 l16 + 7) into `packed`; `other` is lane l16 ^ 8's word.  Key rows take
// the storage order of q4_key_offset.  Value rows put the pair 64g + 4m + 2k, +1
// at byte 4m + 2g + k (word m = d 4m .. 4m+3 of both groups): with j = l16 %
// 8, the low halves of lanes j and j + 8 form word 2j, their high halves word
// 2j+1.
__device__ __forceinline__ void store_q4_row(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                             uint16_t* __restrict__ ks, uint16_t* __restrict__ kz,
                                             uint16_t* __restrict__ vs, uint16_t* __restrict__ vz, int kind,
                                             size_t dst, int l16, uint32_t packed, uint32_t other, uint16_t s16,
                                             uint16_t z16) {
    if (kind == 0) {
        *reinterpret_cast<uint32_t*>(kc + dst * (kHD / 2) + q4_key_offset(l16)) = packed;
    } else {
        const int j = l16 & 7;
        const uint32_t word = (l16 < 8) ? ((packed & 0xFFFFu) | (other << 16))
                                        : ((other >> 16) | (packed & 0xFFFF0000u));
        *reinterpret_cast<uint32_t*>(vc + dst * (kHD / 2) + 4 * (2 * j + (l16 >> 3))) = word;
    }
    if ((l16 & 7) == 0) {
        (kind ? vs : ks)[dst * 2 + (l16 >> 3)] = s16;
        (kind ? vz : kz)[dst * 2 + (l16 >> 3)] = z16;
    }
}

// Re-quantization of aging int8 tokens into the int4 pool ([P4] Sec. 3.3
// practical notes): the int8 row's values code * step (one float32
// multiplication each) go through the write path's group quantizer.  Same
// lane layout as kvq4_quantize_append_kernel; pair `tok` moves int8 slot
// src[tok] to int4 slot dst[tok].  R rows per 16-lane group (loads first):
// 4 for large moves, 1 when a move is small and latency decides.
template <int R>
__global__ __launch_bounds__(256) void kvq4_requantize_q8_kernel(
    uint8_t* __restrict__ kc4, uint8_t* __restrict__ vc4, uint16_t* __restrict__ ks4, uint16_t* __restrict__ kz4,
    uint16_t* __restrict__ vs4, uint16_t* __restrict__ vz4, long n_slots4, const int8_t* __restrict__ kc8,
    const int8_t* __restrict__ vc8, const float* __restrict__ ks8, const float* __restrict__ vs8, long n_slots8,
    DivN nkv, int n_rows, const int32_t* __restrict__ src, const int32_t* __restrict__ dst) {
    const int l16 = threadIdx.x & 15;
    // the slot pairs first, then every row's codes and step
    long s8[R], s4[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int row = min((int)blockIdx.x * (16 * R) + k * 16 + (int)(threadIdx.x >> 4), n_rows - 1);
        const int tok = div_n(row >> 1, nkv);
        s8[k] = src[tok];
        s4[k] = dst[tok];
    }
    uint2 c[R];
    float step[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int row = min((int)blockIdx.x * (16 * R) + k * 16 + (int)(threadIdx.x >> 4), n_rows - 1);
        const int tr = row >> 1;
        const int tok = div_n(tr, nkv);
        // an invalid source reads slot 0 (in bounds) and is not stored
        const long sv = (s8[k] >= 0 && s8[k] < n_slots8) ? s8[k] : 0;
        const int kh = tr - tok * nkv.n;
        const size_t r8 = (size_t)sv * nkv.n + (size_t)kh;
        const size_t c8 = (size_t)sv * nkv.n + (size_t)q8_col(kh, sv, q8_rot_group(nkv.n));
        c[k] = *reinterpret_cast<const uint2*>(((row & 1) ? vc8 : kc8) + c8 * kHD + 8 * l16);
        step[k] = ((row & 1) ? vs8 : ks8)[r8];
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int row = (int)blockIdx.x * (16 * R) + k * 16 + (int)(threadIdx.x >> 4);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sbyte_f(e < 4 ? c[k].x : c[k].y, e & 3) * step[k];
        uint32_t packed;
        uint16_t s16, z16;
        quantize_group8x8(x, packed, s16, z16);
        const uint32_t other = (uint32_t)dpp_i<kDppRowRor8>((int)packed);     // lane l16 ^ 8
        if (row >= n_rows || s8[k] < 0 || s8[k] >= n_slots8 || s4[k] < 0 || s4[k] >= n_slots4) continue;
        const int tr = row >> 1;
        const int tok = div_n(tr, nkv);
        store_q4_row(kc4, vc4, ks4, kz4, vs4, vz4, (int)(row & 1), (size_t)s4[k] * nkv.n + (size_t)(tr - tok * nkv.n),
                     l16, packed, other, s16, z16);
    }
}

}  // namespace kvq

using namespace kvq;

extern "C" int kvq4_quantize_append(uint8_t* k_cache, uint8_t* v_cache, uint16_t* k_scale, uint16_t* k_zero,
                                    uint16_t* v_scale, uint16_t* v_zero, int n_blocks, int kv_bs, int nkv, int hd,
                                    const void* k_new, const void* v_new, int dtype, int n_tokens,
                                    const int32_t* slots, void* stream) {
    if (hd != kHD || !valid_block_size(kv_bs) || nkv < 1 || n_blocks < 1) return KVQ8_ESHAPE;
    if (n_tokens < 0 || dtype < KVQ8_F32 || dtype > KVQ8_F16) return KVQ8_EINVAL;
    if (n_tokens == 0) return KVQ8_OK;
    if (!k_cache || !v_cache || !k_scale || !k_zero || !v_scale || !v_zero || !k_new || !v_new || !slots)
        return KVQ8_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)) return KVQ8_EINVAL;
    const long n_rows = (long)n_tokens * nkv * 2;
    if (n_rows > 0x7FFFFFFFL - kRowsPerBlock) return KVQ8_ESHAPE;
    const long n_slots = (long)n_blocks * kv_bs;
    // pool rows (slot * nkv + head) are 32-bit in the kernel: 2^32 rows would
    // take 256 GiB of codes per cache
    if (n_slots * nkv > 0xFFFFFFFFL) return KVQ8_ESHAPE;
    const uint32_t ns_cap = (uint32_t)(n_slots < 0x80000000L ? n_slots : 0x80000000L);
    const dim3 grid((unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
#define KVQ4_LAUNCH(DT)                                                                                     \
    launch(kvq4_quantize_append_kernel<DT>, grid, block, s, k_cache, v_cache, k_scale, k_zero, \
                       v_scale, v_zero, ns_cap, make_divn(nkv), k_new, v_new, (int)n_rows, slots)
    int st;
    if (dtype == KVQ8_F32) st = KVQ4_LAUNCH(KVQ8_F32);
    else if (dtype == KVQ8_BF16) st = KVQ4_LAUNCH(KVQ8_BF16);
    else st = KVQ4_LAUNCH(KVQ8_F16);
#undef KVQ4_LAUNCH
    return st;
}


extern "C" int kvq4_requantize_q8(uint8_t* k_cache4, uint8_t* v_cache4, uint16_t* k_scale4, uint16_t* k_zero4,
                                  uint16_t* v_scale4, uint16_t* v_zero4, int n_blocks4, const int8_t* k_cache8,
                                  const int8_t* v_cache8, const float* k_scale8, const float* v_scale8, int n_blocks8,
                                  int kv_bs, int nkv, int hd, int n_tokens, const int32_t* src_slots,
                                  const int32_t* dst_slots, void* stream) {
    if (hd != kHD || !valid_block_size(kv_bs) || nkv < 1 || n_blocks4 < 1 || n_blocks8 < 1) return KVQ8_ESHAPE;
    if (n_tokens < 0) return KVQ8_EINVAL;
    if (n_tokens == 0) return KVQ8_OK;
    if (!k_cache4 || !v_cache4 || !k_scale4 || !k_zero4 || !v_scale4 || !v_zero4 || !k_cache8 || !v_cache8 ||
        !k_scale8 || !v_scale8 || !src_slots || !dst_slots)
        return KVQ8_EINVAL;
    if (!aligned16(k_cache4) || !aligned16(v_cache4) || !aligned16(k_cache8) || !aligned16(v_cache8))
        return KVQ8_EINVAL;
    const long n_rows = (long)n_tokens * nkv * 2;
    if (n_rows > 0x7FFFFFFFL - 64) return KVQ8_ESHAPE;       // rows are indexed with 32-bit integers
    const long n_slots4 = (long)n_blocks4 * kv_bs, n_slots8 = (long)n_blocks8 * kv_bs;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int st;
    if (n_rows >= 65536)
        st = launch(kvq4_requantize_q8_kernel<4>, dim3((unsigned)((n_rows + 63) / 64)), dim3(256), s,
                           k_cache4, v_cache4, k_scale4, k_zero4, v_scale4, v_zero4, n_slots4, k_cache8, v_cache8,
                           k_scale8, v_scale8, n_slots8, make_divn(nkv), (int)n_rows, src_slots, dst_slots);
    else
        st = launch(kvq4_requantize_q8_kernel<1>, dim3((unsigned)((n_rows + 15) / 16)), dim3(256), s,
                           k_cache4, v_cache4, k_scale4, k_zero4, v_scale4, v_zero4, n_slots4, k_cache8, v_cache8,
                           k_scale8, v_scale8, n_slots8, make_divn(nkv), (int)n_rows, src_slots, dst_slots);
    return st;
}
