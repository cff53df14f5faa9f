// Write paths of the int4 group variant ([P4] Sec. 3.2 quantizer with the
// Sec. 5.2 checklist; Sec. 3.3 re-quantization of aging int8 tokens).
//
// Both kernels: one (token, kv-head, K-or-V) row per 8 lanes, 16 values per
// lane, R rows per 8-lane group (loads first); each 64-value group is one
// quad, so its max / min need two quad DPP steps (quad_group_codes).  Pairs
// are taken kv-head-major (pair q = kv-head * n + token), so consecutive
// 8-lane groups write consecutive slots of one kv-head: contiguous rows of
// the head-major pool when the slots are consecutive.
#include "kvq8.h"
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

// The lane's 8 output bytes of an int4 row from its code words (byte i of
// cb[h] the code of value 4h + i), written at 16c + 8g.  Key rows: the lane's
// pairs 64g + 16c + 2j go to bytes 16c + 8g + j.  Value rows: the pair 64g +
// 4m + 2k, +1 goes to byte 4m + 2g + k, so words m = 4c .. 4c + 3 take two
// bytes from each lane of the mirror pair; the g = 0 lane writes words 4c,
// 4c + 1, its partner words 4c + 2, 4c + 3.  Every lane of the row takes
// part (DPP).
__device__ __forceinline__ uint2 q4_row_word(const GroupLane& L, uint32_t (&cb)[4]) {
    // (b << 4) | (b >> 8) puts the pairs (c0, c1) and (c2, c3) of a code word
    // in bytes 0 and 2, even element high
#pragma unroll
    for (int h = 0; h < 4; ++h) cb[h] = (cb[h] << 4) | (cb[h] >> 8);
    const uint32_t pk0 = __builtin_amdgcn_perm(cb[1], cb[0], 0x06040200u);   // pairs 0..3
    const uint32_t pk1 = __builtin_amdgcn_perm(cb[3], cb[2], 0x06040200u);   // pairs 4..7
    if (L.kind == 0) return make_uint2(pk0, pk1);
    // the g = 0 lane needs the partner's bytes 0..3, the g = 1 lane the
    // partner's bytes 4..7
    const uint32_t r = (uint32_t)dpp_i<kDppHalfMirror>((int)(L.g ? pk0 : pk1));
    const uint32_t lo = L.g ? r : pk0, hi = L.g ? pk1 : r;
    return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05040100u), __builtin_amdgcn_perm(hi, lo, 0x07060302u));
}

__device__ __forceinline__ void q4_store(const GroupLane& L, uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                         uint16_t* __restrict__ zeros, uint32_t drow, uint2 word, uint16_t s16,
                                         uint16_t z16) {
    *reinterpret_cast<uint2*>(codes + (size_t)drow * (kHD / 2) + 16u * (uint32_t)L.c + 8u * (uint32_t)L.g) = word;
    if (L.c == 0) {
        scales[(size_t)drow * 2 + L.g] = s16;
        zeros[(size_t)drow * 2 + L.g] = z16;
    }
}

constexpr int kRowsPerGroup = 4;            // rows per 8-lane group, loads first
constexpr int kRowsPerBlock = 32 * kRowsPerGroup;

// Pool rows (hm_row) fit in 32 bits (the host checks n_slots * nkv); ns_cap =
// min(n_slots, 2^31) turns the slot test into one unsigned compare.
template <int DT>
__global__ __launch_bounds__(256) void kvq4_quantize_append_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, uint16_t* __restrict__ ks, uint16_t* __restrict__ kz,
    uint16_t* __restrict__ vs, uint16_t* __restrict__ vz, uint32_t ns_cap, int nkv, DivN ntok, int log2_bs,
    const void* __restrict__ k_new, const void* __restrict__ v_new, int n_rows, const int32_t* __restrict__ slots) {
    constexpr int kInBytes = DT == KVQ8_F32 ? 4 : 2;
    const GroupLane L;
    const void* src = L.kind ? v_new : k_new;
    const uint32_t in_off = (uint32_t)(64 * L.g + 16 * L.c) * kInBytes;
    Raw16<DT> raw[kRowsPerGroup];
    int khs[kRowsPerGroup];
    uint32_t slot[kRowsPerGroup];
    // rows past the end load the last row again and store nothing; indices
    // fit in 32 bits (the host checks the row count)
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        const int row = (int)blockIdx.x * kRowsPerBlock + k * 32 + (threadIdx.x >> 3);
        int tok;
        head_major_pair(min(row, n_rows - 1) >> 1, ntok, tok, khs[k]);
        load_raw16<DT>(src, ((size_t)tok * nkv + khs[k]) * (kHD * kInBytes) + in_off, raw[k]);
        slot[k] = (uint32_t)slots[tok];
    }
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        float x[16];
        unpack_raw16<DT>(raw[k], x);
        uint32_t cb[4];
        uint16_t s16, z16;
        quad_group_codes<15>(x, cb, s16, z16);      // every lane of the group takes part (DPP)
        const uint2 word = q4_row_word(L, cb);
        const int row = (int)blockIdx.x * kRowsPerBlock + k * 32 + (threadIdx.x >> 3);
        if (row >= n_rows || slot[k] >= ns_cap) continue;   // uniform per 8-lane row
        q4_store(L, L.kind ? vc : kc, L.kind ? vs : ks, L.kind ? vz : kz,
                 hm_row32(slot[k], (uint32_t)khs[k], (uint32_t)nkv, log2_bs), word, s16, z16);
    }
}

// Re-quantization of aging int8 tokens into the int4 pool ([P4] Sec. 3.3
// practical notes): the int8 row's values code * step (one float32
// multiplication each) go through the write path's group quantizer.  Pair
// i moves int8 slot src[i] to int4 slot dst[i].  R rows per 8-lane group
// (loads first): 4 for large moves, 1 when a move is small and latency
// decides.  The lane reads its 16 codes (16 bytes) of the int8 row.
template <int R>
__global__ __launch_bounds__(256) void kvq4_requantize_q8_kernel(
    uint8_t* __restrict__ kc4, uint8_t* __restrict__ vc4, uint16_t* __restrict__ ks4, uint16_t* __restrict__ kz4,
    uint16_t* __restrict__ vs4, uint16_t* __restrict__ vz4, uint32_t ns4_cap, const int8_t* __restrict__ kc8,
    const int8_t* __restrict__ vc8, const float* __restrict__ ks8, const float* __restrict__ vs8,
    uint32_t ns8_cap, int nkv, DivN npairs, int log2_bs, int n_rows, const int32_t* __restrict__ src,
    const int32_t* __restrict__ dst) {
    const GroupLane L;
    const int rot = q8_rot_group(nkv);
    // the slot pairs first, then every row's codes and step
    uint32_t s8[R], s4[R];
    int khs[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int row = (int)blockIdx.x * (32 * R) + k * 32 + (int)(threadIdx.x >> 3);
        int i;
        head_major_pair(min(row, n_rows - 1) >> 1, npairs, i, khs[k]);
        s8[k] = (uint32_t)src[i];
        s4[k] = (uint32_t)dst[i];
    }
    uint4 cw[R];
    float step[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        // an invalid source reads slot 0 (in bounds) and is not stored
        const uint32_t sv = s8[k] < ns8_cap ? s8[k] : 0u;
        const size_t r8 = (size_t)sv * nkv;
        const size_t c8 = r8 + (size_t)q8_col(khs[k], sv, rot);
        cw[k] = *reinterpret_cast<const uint4*>((L.kind ? vc8 : kc8) + c8 * kHD + 64 * L.g + 16 * L.c);
        step[k] = (L.kind ? vs8 : ks8)[r8 + (size_t)khs[k]];
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const uint32_t w[4] = {cw[k].x, cw[k].y, cw[k].z, cw[k].w};
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = sbyte_f(w[e >> 2], e & 3) * step[k];
        uint32_t cb[4];
        uint16_t s16, z16;
        quad_group_codes<15>(x, cb, s16, z16);
        const uint2 word = q4_row_word(L, cb);
        const int row = (int)blockIdx.x * (32 * R) + k * 32 + (int)(threadIdx.x >> 3);
        if (row >= n_rows || s8[k] >= ns8_cap || s4[k] >= ns4_cap) continue;   // uniform per 8-lane row
        q4_store(L, L.kind ? vc4 : kc4, L.kind ? vs4 : ks4, L.kind ? vz4 : kz4,
                 hm_row32(s4[k], (uint32_t)khs[k], (uint32_t)nkv, log2_bs), word, s16, z16);
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
    // pool rows are 32-bit in the kernel: 2^32 rows would take 256 GiB of
    // codes per cache
    if (n_slots * nkv > 0xFFFFFFFFL) return KVQ8_ESHAPE;
    const dim3 grid((unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
#define KVQ4_LAUNCH(DT)                                                                                    \
    launch(kvq4_quantize_append_kernel<DT>, grid, block, s, k_cache, v_cache, k_scale, k_zero, v_scale, v_zero, \
           slot_cap(n_slots), nkv, make_divn(n_tokens), ilog2(kv_bs), k_new, v_new, (int)n_rows, slots)
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
    if (n_rows > 0x7FFFFFFFL - 128) return KVQ8_ESHAPE;      // rows are indexed with 32-bit integers
    const long n_slots4 = (long)n_blocks4 * kv_bs, n_slots8 = (long)n_blocks8 * kv_bs;
    if (n_slots4 * nkv > 0xFFFFFFFFL) return KVQ8_ESHAPE;   // 32-bit int4 pool rows
    hipStream_t s = static_cast<hipStream_t>(stream);
    int st;
    if (n_rows >= 65536)
        st = launch(kvq4_requantize_q8_kernel<4>, dim3((unsigned)((n_rows + 127) / 128)), dim3(256), s, k_cache4,
                    v_cache4, k_scale4, k_zero4, v_scale4, v_zero4, slot_cap(n_slots4), k_cache8, v_cache8, k_scale8,
                    v_scale8, slot_cap(n_slots8), nkv, make_divn(n_tokens), ilog2(kv_bs), (int)n_rows, src_slots,
                    dst_slots);
    else
        st = launch(kvq4_requantize_q8_kernel<1>, dim3((unsigned)((n_rows + 31) / 32)), dim3(256), s, k_cache4,
                    v_cache4, k_scale4, k_zero4, v_scale4, v_zero4, slot_cap(n_slots4), k_cache8, v_cache8, k_scale8,
                    v_scale8, slot_cap(n_slots8), nkv, make_divn(n_tokens), ilog2(kv_bs), (int)n_rows, src_slots,
                    dst_slots);
    return st;
}
