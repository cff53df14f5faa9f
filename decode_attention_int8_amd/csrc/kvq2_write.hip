// Write paths of the 2-bit band ([P4] Sec. 3.2 group quantizer at two bits,
// Sec. 3.3 re-quantization of aging blocks).
//
// The 2-bit row layouts: key word 2g + h holds d = 64h + 16g + 4k + j at bits
// 8j + 2k; the value row's 16-bit word m holds d = 64(s/4) + 4m + s%4 at bits
// 2s.
//
// kvq2_quantize_append_kernel: the int4 append kernel's lanes, one row per 8
// lanes, lane l holding elements 64g + 16c .. + 15 (g = l / 4; c = l % 4, or
// 3 - l % 4 for g = 1), so a lane's 16 codes are key word 2c + g, and its
// value bytes meet those of lane 7 - l (the other group, same c) in words
// 4c .. 4c + 3.
// kvq2_requantize_q4_kernel: one row per 16 lanes, 8 values per lane
// (elements 8 l16 .. 8 l16 + 7), each group an aligned 8-lane half row: lanes
// 2w and 2w + 1 of a half row fill key word w = 2g + h between them; lane j of
// the low half and lane j + 8 of the high half fill value words 2j and 2j + 1.
#include "kvq8.h"
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

constexpr int kRow2Bytes = kHD / 4;
constexpr int kRows2PerGroup = 4;             // rows per 8-lane group, loads first
constexpr int kRows2PerBlock = 32 * kRows2PerGroup;

// Quantize the lane's 8 values of a 64-value group held by an aligned 8-lane
// half row to 2-bit codes: scale = (max - min) / 3 (1 for a constant group),
// floored at 1e-7 and rounded to binary16 before use; zero = rint(-min / s)
// clamped to [0, 3]; code = clamp(rint(x / s + zero), 0, 3).  Returns the
// codes (2 bits each, element e at bits 2e) and the binary16 scale and zero.
__device__ __forceinline__ void quantize_group8x8_q2(const float (&x)[8], uint32_t& codes, uint16_t& s16,
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
    float s32 = (mx == mn) ? 1.0f : (mx - mn) / 3.0f;
    s32 = fmaxf(s32, 1e-7f);
    s16 = __builtin_bit_cast(uint16_t, (_Float16)s32);
    const float s = half_bits_f(s16);
    // integer zero point in [0, 3]; + 0.0f stores a zero as +0.0
    const float z = fminf(fmaxf(rintf(-mn / s), 0.0f), 3.0f) + 0.0f;
    z16 = __builtin_bit_cast(uint16_t, (_Float16)z);
    const float rs = __builtin_amdgcn_rcpf(s);
    // code = clamp(rint(x / s + z), 0, 3) with z an integer, the quotient
    // computed only near a half-integer.  Elsewhere the clamped q + z plus
    // 1.5 * 2^23 holds rint(q + z) in its low byte (the addition rounds half
    // to even like rint); the codes are gathered by byte permutes and a dot
    // product with (1, 4, 16, 64).
    constexpr float kMagic = 12582912.0f;
    uint32_t cb[8];
    bool slow[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float q = x[e] * rs;
        slow[e] = near_half(q);
        cb[e] = __float_as_uint(__builtin_amdgcn_fmed3f(q + z, 0.0f, 3.0f) + kMagic);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (__builtin_amdgcn_ballot_w64(slow[e]) != 0) {      // rare: one wave-uniform test per value
            const float cd = fminf(fmaxf(rintf(x[e] / s + z), 0.0f), 3.0f);
            cb[e] = slow[e] ? (uint32_t)(int)cd : cb[e];
        }
    }
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t b = __builtin_amdgcn_perm(cb[4 * h + 1], cb[4 * h], 0x0C0C0400u) |
                           __builtin_amdgcn_perm(cb[4 * h + 3], cb[4 * h + 2], 0x04000C0Cu);
        w[h] = __builtin_amdgcn_udot4(b, 0x40100401u, 0u, false);     // c0 + 4 c1 + 16 c2 + 64 c3
    }
    codes = w[0] | (w[1] << 8);
}

// Store one row.  Lane l16 holds elements 8 l16 + e: group h = l16 / 8, and
// within the group d' = 8 (l16 % 8) + e.
//   key:   d' = 16g + 4k + j with g = (l16 % 8) / 2, k = 2 (l16 % 2) + e / 4,
//          j = e % 4; word 2g + h, bit 8j + 2k.  The lane's part of the word
//          and its neighbour's (l16 ^ 1) are OR-ed; the even lane stores.
//   value: d' = 4m + r with m = 2 (l16 % 8) + e / 4, r = e % 4; 16-bit word m,
//          bit 2 (4h + r).  Lanes j and j + 8 (groups 0 and 1) fill the two
//          words 2j, 2j + 1; lane j stores.
__device__ __forceinline__ void store_q2_row(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                             uint16_t* __restrict__ ks, uint16_t* __restrict__ kz,
                                             uint16_t* __restrict__ vs, uint16_t* __restrict__ vz, int kind,
                                             size_t dst, int l16, uint32_t kpart, uint32_t kother, uint32_t vpart,
                                             uint32_t vother, uint16_t s16, uint16_t z16) {
    if (kind == 0) {
        if ((l16 & 1) == 0) {
            const int g = (l16 & 7) >> 1, h = l16 >> 3;
            *reinterpret_cast<uint32_t*>(kc + dst * kRow2Bytes + 4 * (2 * g + h)) = kpart | kother;
        }
    } else {
        if (l16 < 8) *reinterpret_cast<uint32_t*>(vc + dst * kRow2Bytes + 4 * l16) = vpart | vother;
    }
    if ((l16 & 7) == 0) {
        (kind ? vs : ks)[dst * 2 + (l16 >> 3)] = s16;
        (kind ? vz : kz)[dst * 2 + (l16 >> 3)] = z16;
    }
}

// The lane's parts of the key and value words from its 8 codes (element e at
// bits 2e of `codes`).
__device__ __forceinline__ void q2_parts(uint32_t codes, int l16, uint32_t& kpart, uint32_t& vpart) {
    uint32_t kp = 0, vp = 0;
    const int kk = 2 * (l16 & 1);
    const int h = l16 >> 3;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t c = (codes >> (2 * e)) & 3u;
        kp |= c << (8 * (e & 3) + 2 * (kk + (e >> 2)));
        vp |= c << (16 * (e >> 2) + 2 * (4 * h + (e & 3)));
    }
    kpart = kp;
    vpart = vp;
}

// Row numbers of the pool (slot * nkv + head) fit in 32 bits (the host checks
// n_slots * nkv; ns_cap = min(n_slots, 2^31)).
template <int DT>
__global__ __launch_bounds__(256) void kvq2_quantize_append_kernel(
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
    // key word 2c + g; value words 4c + 2g, 4c + 2g + 1 (bytes 8c + 4g ..)
    const uint32_t out_off = kind ? 8u * (uint32_t)c + 4u * (uint32_t)g : 4u * (uint32_t)(2 * c + g);
    // value bytes of words 4c + 2g, + 1: [own v(2g), partner v(2g), own
    // v(2g + 1), partner v(2g + 1)] with the group 0 byte low in each word
    const uint32_t vsel = g ? 0x03070206u : 0x05010400u;
    uint8_t* codes = kind ? vc : kc;
    uint16_t* scales = kind ? vs : ks;
    uint16_t* zeros = kind ? vz : kz;
    Raw16<DT> raw[kRows2PerGroup];
    int trs[kRows2PerGroup];
    uint32_t slot[kRows2PerGroup];
    // rows past the end load the last row again and store nothing; indices
    // fit in 32 bits (the host checks the row count)
#pragma unroll
    for (int k = 0; k < kRows2PerGroup; ++k) {
        const int row = (int)blockIdx.x * kRows2PerBlock + k * 32 + (threadIdx.x >> 3);
        const int tr = min(row, n_rows - 1) >> 1;  // token * nkv + kv-head
        trs[k] = tr;
        load_raw16<DT>(src, (size_t)tr * (kHD * kInBytes) + in_off, raw[k]);
        slot[k] = (uint32_t)slots[div_n(tr, nkv)];
    }
#pragma unroll
    for (int k = 0; k < kRows2PerGroup; ++k) {
        float x[16];
        unpack_raw16<DT>(raw[k], x);
        uint32_t cb[4];
        uint16_t s16, z16;
        quad_group_codes<3>(x, cb, s16, z16);       // every lane of the group takes part (DPP)
        uint32_t word;
        if (kind == 0) {
            // element t = 4k + j of the lane at bits 8j + 2k: byte j of code
            // word k, shifted by 2k
            word = cb[0] | (cb[1] << 2) | (cb[2] << 4) | (cb[3] << 6);
        } else {
            // value byte i = codes 4i .. 4i + 3 at bits 0, 2, 4, 6
            uint32_t v = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) v |= __builtin_amdgcn_udot4(cb[i], 0x40100401u, 0u, false) << (8 * i);
            const uint32_t r = (uint32_t)dpp_i<kDppHalfMirror>((int)v);   // the other group's lane
            word = __builtin_amdgcn_perm(r, v, vsel);
        }
        const int row = (int)blockIdx.x * kRows2PerBlock + k * 32 + (threadIdx.x >> 3);
        if (row >= n_rows || slot[k] >= ns_cap) continue;   // uniform per 8-lane row
        const uint32_t drow = slot[k] * (uint32_t)nkv.n + (uint32_t)(trs[k] - div_n(trs[k], nkv) * nkv.n);
        *reinterpret_cast<uint32_t*>(codes + (size_t)drow * kRow2Bytes + out_off) = word;
        if (c == 0) {
            scales[(size_t)drow * 2 + g] = s16;
            zeros[(size_t)drow * 2 + g] = z16;
        }
    }
}

// Re-quantization of aging int4 tokens into the 2-bit pool: the int4 row's
// values (code - zero) * scale (exact in float32) go through the 2-bit group
// quantizer.  Pair `tok` moves int4 slot src[tok] to 2-bit slot dst[tok].  R
// rows per 16-lane group (loads first): 4 for large moves, 1 for small ones.
// The int4 rows are read in their layouts: key bytes 4 l16 .. 4 l16 + 3 hold
// the lane's 8 codes (even element in the high nibble); value bytes 8j + 2h,
// + 1 and 8j + 4 + 2h, + 1 (j = l16 % 8) hold elements 64h + 8j .. + 3 and
// + 4 .. + 7.
template <int R>
__global__ __launch_bounds__(256) void kvq2_requantize_q4_kernel(
    uint8_t* __restrict__ kc2, uint8_t* __restrict__ vc2, uint16_t* __restrict__ ks2, uint16_t* __restrict__ kz2,
    uint16_t* __restrict__ vs2, uint16_t* __restrict__ vz2, long n_slots2, const uint8_t* __restrict__ kc4,
    const uint8_t* __restrict__ vc4, const uint16_t* __restrict__ ks4, const uint16_t* __restrict__ kz4,
    const uint16_t* __restrict__ vs4, const uint16_t* __restrict__ vz4, long n_slots4, DivN nkv, int n_rows,
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst) {
    const int l16 = threadIdx.x & 15;
    const int h = l16 >> 3;
    const int j = l16 & 7;
    long s4[R], s2[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int row = min((int)blockIdx.x * (16 * R) + k * 16 + (int)(threadIdx.x >> 4), n_rows - 1);
        const int tok = div_n(row >> 1, nkv);
        s4[k] = src[tok];
        s2[k] = dst[tok];
    }
    uint32_t c0[R], c1[R];
    uint16_t sc[R], zp[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int row = min((int)blockIdx.x * (16 * R) + k * 16 + (int)(threadIdx.x >> 4), n_rows - 1);
        const int tr = row >> 1;
        const int tok = div_n(tr, nkv);
        // an invalid source reads slot 0 (in bounds) and is not stored
        const long sv = (s4[k] >= 0 && s4[k] < n_slots4) ? s4[k] : 0;
        const size_t r4 = (size_t)sv * nkv.n + (size_t)(tr - tok * nkv.n);
        if (row & 1) {
            c0[k] = *reinterpret_cast<const uint32_t*>(vc4 + r4 * (kHD / 2) + 8 * j);
            c1[k] = *reinterpret_cast<const uint32_t*>(vc4 + r4 * (kHD / 2) + 8 * j + 4);
            sc[k] = vs4[r4 * 2 + h];
            zp[k] = vz4[r4 * 2 + h];
        } else {
            c0[k] = *reinterpret_cast<const uint32_t*>(kc4 + r4 * (kHD / 2) + q4_key_offset(l16));
            c1[k] = 0u;
            sc[k] = ks4[r4 * 2 + h];
            zp[k] = kz4[r4 * 2 + h];
        }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int row = (int)blockIdx.x * (16 * R) + k * 16 + (int)(threadIdx.x >> 4);
        const int rr = min(row, n_rows - 1);
        // the lane's 8 int4 codes, element e in bits 4e (pairs: even element high)
        uint32_t pairs;
        if (rr & 1) {
            // value: the 16 bits at 2h of each word hold elements (0,1), (2,3)
            // and (4,5), (6,7)
            pairs = ((c0[k] >> (16 * h)) & 0xFFFFu) | (((c1[k] >> (16 * h)) & 0xFFFFu) << 16);
        } else {
            pairs = c0[k];
        }
        const float s = half_bits_f(sc[k]);
        const float z = half_bits_f(zp[k]);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t byte = (pairs >> (8 * (e >> 1))) & 0xFFu;
            const uint32_t code = (e & 1) ? (byte & 0xFu) : (byte >> 4);
            x[e] = ((float)code - z) * s;
        }
        uint32_t codes, kpart, vpart;
        uint16_t s16, z16;
        quantize_group8x8_q2(x, codes, s16, z16);
        q2_parts(codes, l16, kpart, vpart);
        const uint32_t kother = (uint32_t)dpp_i<kDppXor1>((int)kpart);
        const uint32_t vother = (uint32_t)dpp_i<kDppRowRor8>((int)vpart);
        if (row >= n_rows || s4[k] < 0 || s4[k] >= n_slots4 || s2[k] < 0 || s2[k] >= n_slots2) continue;
        const int tr = row >> 1;
        const int tok = div_n(tr, nkv);
        store_q2_row(kc2, vc2, ks2, kz2, vs2, vz2, (int)(row & 1),
                     (size_t)s2[k] * nkv.n + (size_t)(tr - tok * nkv.n), l16, kpart, kother, vpart, vother, s16,
                     z16);
    }
}

}  // namespace kvq

using namespace kvq;

extern "C" int kvq2_quantize_append(uint8_t* k_cache, uint8_t* v_cache, uint16_t* k_scale, uint16_t* k_zero,
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
    if (n_rows > 0x7FFFFFFFL - kRows2PerBlock) return KVQ8_ESHAPE;
    const long n_slots = (long)n_blocks * kv_bs;
    // pool rows (slot * nkv + head) are 32-bit in the kernel: 2^32 rows would
    // take 160 GiB per cache (codes, scales and zeros)
    if (n_slots * nkv > 0xFFFFFFFFL) return KVQ8_ESHAPE;
    const uint32_t ns_cap = (uint32_t)(n_slots < 0x80000000L ? n_slots : 0x80000000L);
    const dim3 grid((unsigned)((n_rows + kRows2PerBlock - 1) / kRows2PerBlock)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
#define KVQ2_LAUNCH(DT)                                                                                     \
    launch(kvq2_quantize_append_kernel<DT>, grid, block, s, k_cache, v_cache, k_scale, k_zero, \
                       v_scale, v_zero, ns_cap, make_divn(nkv), k_new, v_new, (int)n_rows, slots)
    int st;
    if (dtype == KVQ8_F32) st = KVQ2_LAUNCH(KVQ8_F32);
    else if (dtype == KVQ8_BF16) st = KVQ2_LAUNCH(KVQ8_BF16);
    else st = KVQ2_LAUNCH(KVQ8_F16);
#undef KVQ2_LAUNCH
    return st;
}

extern "C" int kvq2_requantize_q4(uint8_t* k_cache2, uint8_t* v_cache2, uint16_t* k_scale2, uint16_t* k_zero2,
                                  uint16_t* v_scale2, uint16_t* v_zero2, int n_blocks2, const uint8_t* k_cache4,
                                  const uint8_t* v_cache4, const uint16_t* k_scale4, const uint16_t* k_zero4,
                                  const uint16_t* v_scale4, const uint16_t* v_zero4, int n_blocks4, int kv_bs,
                                  int nkv, int hd, int n_tokens, const int32_t* src_slots, const int32_t* dst_slots,
                                  void* stream) {
    if (hd != kHD || !valid_block_size(kv_bs) || nkv < 1 || n_blocks2 < 1 || n_blocks4 < 1) return KVQ8_ESHAPE;
    if (n_tokens < 0) return KVQ8_EINVAL;
    if (n_tokens == 0) return KVQ8_OK;
    if (!k_cache2 || !v_cache2 || !k_scale2 || !k_zero2 || !v_scale2 || !v_zero2 || !k_cache4 || !v_cache4 ||
        !k_scale4 || !k_zero4 || !v_scale4 || !v_zero4 || !src_slots || !dst_slots)
        return KVQ8_EINVAL;
    if (!aligned16(k_cache2) || !aligned16(v_cache2) || !aligned16(k_cache4) || !aligned16(v_cache4))
        return KVQ8_EINVAL;
    const long n_rows = (long)n_tokens * nkv * 2;
    if (n_rows > 0x7FFFFFFFL - 64) return KVQ8_ESHAPE;       // rows are indexed with 32-bit integers
    const long n_slots2 = (long)n_blocks2 * kv_bs, n_slots4 = (long)n_blocks4 * kv_bs;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int st;
    if (n_rows >= 65536)
        st = launch(kvq2_requantize_q4_kernel<4>, dim3((unsigned)((n_rows + 63) / 64)), dim3(256), s,
                           k_cache2, v_cache2, k_scale2, k_zero2, v_scale2, v_zero2, n_slots2, k_cache4, v_cache4,
                           k_scale4, k_zero4, v_scale4, v_zero4, n_slots4, make_divn(nkv), (int)n_rows, src_slots,
                           dst_slots);
    else
        st = launch(kvq2_requantize_q4_kernel<1>, dim3((unsigned)((n_rows + 15) / 16)), dim3(256), s,
                           k_cache2, v_cache2, k_scale2, k_zero2, v_scale2, v_zero2, n_slots2, k_cache4, v_cache4,
                           k_scale4, k_zero4, v_scale4, v_zero4, n_slots4, make_divn(nkv), (int)n_rows, src_slots,
                           dst_slots);
    return st;
}
