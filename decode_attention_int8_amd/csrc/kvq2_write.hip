// Write paths of the 2-bit band ([P4] Sec. 3.2 group quantizer at two bits,
// Sec. 3.3 re-quantization of aging blocks).
//
// The 2-bit row layouts: key word 2g + h holds d = 64h + 16g + 4k + j at bits
// 8j + 2k; the value row's 16-bit word m holds d = 64(s/4) + 4m + s%4 at bits
// 2s.
//
// Both kernels use the int4 write kernels' lanes (GroupLane: one row per 8
// lanes, lane l holding elements 64g + 16c .. + 15) and their kv-head-major
// pair order.  A lane's 16 codes are then key word 2c + g, and its value
// bytes meet those of lane 7 - l (the other group, same c) in words 4c ..
// 4c + 3.
#include "kvq8.h"
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

constexpr int kRow2Bytes = kHD / 4;
constexpr int kRows2PerGroup = 4;             // rows per 8-lane group, loads first
constexpr int kRows2PerBlock = 32 * kRows2PerGroup;

// The lane's 32-bit word of a 2-bit row from its code words (byte i of cb[h]
// the code of value 4h + i), written at byte q2_out_off: the key word 2c + g,
// or the value bytes of words 4c + 2g, 4c + 2g + 1.  Every lane of the row
// takes part (DPP).
__device__ __forceinline__ uint32_t q2_row_word(const GroupLane& L, const uint32_t (&cb)[4]) {
    if (L.kind == 0) {
        // element t = 4k + j of the lane at bits 8j + 2k: byte j of code
        // word k, shifted by 2k
        return cb[0] | (cb[1] << 2) | (cb[2] << 4) | (cb[3] << 6);
    }
    // value byte i = codes 4i .. 4i + 3 at bits 0, 2, 4, 6
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) v |= __builtin_amdgcn_udot4(cb[i], 0x40100401u, 0u, false) << (8 * i);
    const uint32_t r = (uint32_t)dpp_i<kDppHalfMirror>((int)v);   // the other group's lane
    // words 4c + 2g, + 1: [v(2g) of group 0, of group 1, v(2g + 1) of group 0,
    // of group 1], the group 0 byte low in each word
    return __builtin_amdgcn_perm(r, v, L.g ? 0x03070206u : 0x05010400u);
}

__device__ __forceinline__ void q2_store(const GroupLane& L, uint8_t* __restrict__ codes,
                                         uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, uint32_t drow,
                                         uint32_t word, uint16_t s16, uint16_t z16) {
    const uint32_t off = L.kind ? 8u * (uint32_t)L.c + 4u * (uint32_t)L.g : 4u * (uint32_t)(2 * L.c + L.g);
    *reinterpret_cast<uint32_t*>(codes + (size_t)drow * kRow2Bytes + off) = word;
    if (L.c == 0) {
        scales[(size_t)drow * 2 + L.g] = s16;
        zeros[(size_t)drow * 2 + L.g] = z16;
    }
}

// Pool rows (hm_row) fit in 32 bits (the host checks n_slots * nkv); ns_cap =
// min(n_slots, 2^31) turns the slot test into one unsigned compare.
template <int DT>
__global__ __launch_bounds__(256) void kvq2_quantize_append_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, uint16_t* __restrict__ ks, uint16_t* __restrict__ kz,
    uint16_t* __restrict__ vs, uint16_t* __restrict__ vz, uint32_t ns_cap, int nkv, DivN ntok, int log2_bs,
    const void* __restrict__ k_new, const void* __restrict__ v_new, int n_rows, const int32_t* __restrict__ slots) {
    constexpr int kInBytes = DT == KVQ8_F32 ? 4 : 2;
    const GroupLane L;
    const void* src = L.kind ? v_new : k_new;
    const uint32_t in_off = (uint32_t)(64 * L.g + 16 * L.c) * kInBytes;
    Raw16<DT> raw[kRows2PerGroup];
    int khs[kRows2PerGroup];
    uint32_t slot[kRows2PerGroup];
    // rows past the end load the last row again and store nothing; indices
    // fit in 32 bits (the host checks the row count)
#pragma unroll
    for (int k = 0; k < kRows2PerGroup; ++k) {
        const int row = (int)blockIdx.x * kRows2PerBlock + k * 32 + (threadIdx.x >> 3);
        int tok;
        head_major_pair(min(row, n_rows - 1) >> 1, ntok, tok, khs[k]);
        load_raw16<DT>(src, ((size_t)tok * nkv + khs[k]) * (kHD * kInBytes) + in_off, raw[k]);
        slot[k] = (uint32_t)slots[tok];
    }
#pragma unroll
    for (int k = 0; k < kRows2PerGroup; ++k) {
        float x[16];
        unpack_raw16<DT>(raw[k], x);
        uint32_t cb[4];
        uint16_t s16, z16;
        quad_group_codes<3>(x, cb, s16, z16);       // every lane of the group takes part (DPP)
        const uint32_t word = q2_row_word(L, cb);
        const int row = (int)blockIdx.x * kRows2PerBlock + k * 32 + (threadIdx.x >> 3);
        if (row >= n_rows || slot[k] >= ns_cap) continue;   // uniform per 8-lane row
        q2_store(L, L.kind ? vc : kc, L.kind ? vs : ks, L.kind ? vz : kz,
                 hm_row32(slot[k], (uint32_t)khs[k], (uint32_t)nkv, log2_bs), word, s16, z16);
    }
}

// Re-quantization of aging int4 tokens into the 2-bit pool: the int4 row's
// values (code - zero) * scale (exact in float32) go through the 2-bit group
// quantizer.  Pair i moves int4 slot src[i] to 2-bit slot dst[i].  R rows
// per 8-lane group (loads first): 4 for large moves, 1 for small ones.  The
// lane's 16 int4 codes, as pairs with the even element in the high nibble,
// are bytes 16c + 8g .. + 7 of a key row, and the halves 2g of the words at
// 16c .. 16c + 15 of a value row.
template <int R>
__global__ __launch_bounds__(256) void kvq2_requantize_q4_kernel(
    uint8_t* __restrict__ kc2, uint8_t* __restrict__ vc2, uint16_t* __restrict__ ks2, uint16_t* __restrict__ kz2,
    uint16_t* __restrict__ vs2, uint16_t* __restrict__ vz2, uint32_t ns2_cap, const uint8_t* __restrict__ kc4,
    const uint8_t* __restrict__ vc4, const uint16_t* __restrict__ ks4, const uint16_t* __restrict__ kz4,
    const uint16_t* __restrict__ vs4, const uint16_t* __restrict__ vz4, uint32_t ns4_cap, int nkv, DivN npairs,
    int log2_bs, int n_rows, const int32_t* __restrict__ src, const int32_t* __restrict__ dst) {
    const GroupLane L;
    uint32_t s4[R], s2[R];
    int khs[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int row = (int)blockIdx.x * (32 * R) + k * 32 + (int)(threadIdx.x >> 3);
        int i;
        head_major_pair(min(row, n_rows - 1) >> 1, npairs, i, khs[k]);
        s4[k] = (uint32_t)src[i];
        s2[k] = (uint32_t)dst[i];
    }
    uint4 cw[R];
    uint16_t sc[R], zp[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        // an invalid source reads slot 0 (in bounds) and is not stored
        const uint32_t r4 = hm_row32(s4[k] < ns4_cap ? s4[k] : 0u, (uint32_t)khs[k], (uint32_t)nkv, log2_bs);
        if (L.kind == 0) {
            const uint2 w = *reinterpret_cast<const uint2*>(kc4 + (size_t)r4 * (kHD / 2) + 16 * L.c + 8 * L.g);
            cw[k] = make_uint4(w.x, w.y, 0u, 0u);
        } else {
            cw[k] = *reinterpret_cast<const uint4*>(vc4 + (size_t)r4 * (kHD / 2) + 16 * L.c);
        }
        sc[k] = (L.kind ? vs4 : ks4)[(size_t)r4 * 2 + L.g];
        zp[k] = (L.kind ? vz4 : kz4)[(size_t)r4 * 2 + L.g];
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
        // the lane's 8 pair bytes, pair j in byte j (even element high)
        uint32_t p0 = cw[k].x, p1 = cw[k].y;
        if (L.kind != 0) {
            const uint32_t sel = L.g ? 0x07060302u : 0x05040100u;   // half 2g of each word
            p0 = __builtin_amdgcn_perm(cw[k].y, cw[k].x, sel);
            p1 = __builtin_amdgcn_perm(cw[k].w, cw[k].z, sel);
        }
        const float s = half_bits_f(sc[k]);
        const float z = half_bits_f(zp[k]);
        float x[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t byte = ((j < 4 ? p0 : p1) >> (8 * (j & 3))) & 0xFFu;
            x[2 * j] = ((float)(byte >> 4) - z) * s;
            x[2 * j + 1] = ((float)(byte & 0xFu) - z) * s;
        }
        uint32_t cb[4];
        uint16_t s16, z16;
        quad_group_codes<3>(x, cb, s16, z16);
        const uint32_t word = q2_row_word(L, cb);
        const int row = (int)blockIdx.x * (32 * R) + k * 32 + (int)(threadIdx.x >> 3);
        if (row >= n_rows || s4[k] >= ns4_cap || s2[k] >= ns2_cap) continue;   // uniform per 8-lane row
        q2_store(L, L.kind ? vc2 : kc2, L.kind ? vs2 : ks2, L.kind ? vz2 : kz2,
                 hm_row32(s2[k], (uint32_t)khs[k], (uint32_t)nkv, log2_bs), word, s16, z16);
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
    // pool rows are 32-bit in the kernel: 2^32 rows would take 160 GiB per
    // cache (codes, scales and zeros)
    if (n_slots * nkv > 0xFFFFFFFFL) return KVQ8_ESHAPE;
    const dim3 grid((unsigned)((n_rows + kRows2PerBlock - 1) / kRows2PerBlock)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
#define KVQ2_LAUNCH(DT)                                                                                    \
    launch(kvq2_quantize_append_kernel<DT>, grid, block, s, k_cache, v_cache, k_scale, k_zero, v_scale, v_zero, \
           slot_cap(n_slots), nkv, make_divn(n_tokens), ilog2(kv_bs), k_new, v_new, (int)n_rows, slots)
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
    if (n_rows > 0x7FFFFFFFL - 128) return KVQ8_ESHAPE;      // rows are indexed with 32-bit integers
    const long n_slots2 = (long)n_blocks2 * kv_bs, n_slots4 = (long)n_blocks4 * kv_bs;
    if (n_slots2 * nkv > 0xFFFFFFFFL || n_slots4 * nkv > 0xFFFFFFFFL) return KVQ8_ESHAPE;   // 32-bit pool rows
    hipStream_t s = static_cast<hipStream_t>(stream);
    int st;
    if (n_rows >= 65536)
        st = launch(kvq2_requantize_q4_kernel<4>, dim3((unsigned)((n_rows + 127) / 128)), dim3(256), s, k_cache2,
                    v_cache2, k_scale2, k_zero2, v_scale2, v_zero2, slot_cap(n_slots2), k_cache4, v_cache4, k_scale4,
                    k_zero4, v_scale4, v_zero4, slot_cap(n_slots4), nkv, make_divn(n_tokens), ilog2(kv_bs),
                    (int)n_rows, src_slots, dst_slots);
    else
        st = launch(kvq2_requantize_q4_kernel<1>, dim3((unsigned)((n_rows + 31) / 32)), dim3(256), s, k_cache2,
                    v_cache2, k_scale2, k_zero2, v_scale2, v_zero2, slot_cap(n_slots2), k_cache4, v_cache4, k_scale4,
                    k_zero4, v_scale4, v_zero4, slot_cap(n_slots4), nkv, make_divn(n_tokens), ilog2(kv_bs),
                    (int)n_rows, src_slots, dst_slots);
    return st;
}
