// Device building blocks shared by the kernels of the int8 / int4 KV library
// (gfx950, wave64).  Cross-lane traffic uses DPP row operations, which the
// compiler fuses into the consuming VALU instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq8.h"

namespace kvq {

constexpr int kHD = 128;        // head dimension
constexpr int kWave = 64;       // wavefront width on CDNA
constexpr int kQBlock = 32;     // query quantization block ([P3] Sec. 2 seg. 1)
constexpr int kTile = 64;       // tokens per wave tile in the decode kernels

// DPP controls (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i inside each 8-lane half row
constexpr int kDppRowRor8 = 0x128;    // lane i <- lane (i+8) mod 16 inside each 16-lane row
constexpr int kDppRowRor4 = 0x124;    // rotation of each 16-lane row by 4 lanes (either way: used where
                                      // only the set of lanes 4 apart matters)
constexpr int kDppQuadRot1 = 0x39;    // quad_perm [1,2,3,0]: lane q <- lane (q+1) mod 4
constexpr int kDppQuadRot3 = 0x93;    // quad_perm [3,0,1,2]: lane q <- lane (q+3) mod 4

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// value from lane (lane ^ 16), within each half of the wave
__device__ __forceinline__ float swz_xor16(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
// value from lane (lane ^ 32)
__device__ __forceinline__ float xor32(float v) {
    const int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(v)));
}

// Reductions over the 8 groups of 8 lanes that hold the same value pattern
// (lanes with equal lane % 8).  Every lane receives the result.
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, dpp_f<kDppRowRor8>(v));
    v = fmaxf(v, swz_xor16(v));
    v = fmaxf(v, xor32(v));
    return v;
}

// signed byte k of a packed dword as float (one SDWA convert)
__device__ __forceinline__ float sbyte_f(uint32_t w, int k) {
    return (float)(int8_t)(w >> (8 * k));
}

// -----------------------------------------------------------------------------
// Query quantization ([P3] Sec. 2 seg. 1) of up to 8 query rows by a
// workgroup of at least 256 threads, into LDS:
//   qm  = max |q| over the 32-value block (qm < 1e-6 -> 1)
//   qsc = qm * (1/127)         (float32 constant 1/127)
//   iq  = 127 / qm             (IEEE division)
//   code= roundf(q * iq) clamped to [-128, 127]
// Thread t handles values 4(t%32) .. +3 of row t/32; the 8 threads of a
// 32-block find its max with three DPP steps.  load_q4 issues the thread's
// load (so that callers can put other loads behind it); quantize_q4 takes
// the loaded values.  Every decode path and the query export use these.
// -----------------------------------------------------------------------------
constexpr int kMaxRows = 8;

struct QSmem {
    uint32_t qc[kMaxRows][kHD / 4];       // codes, 4 per word (little endian)
    float qs[kMaxRows][kHD / kQBlock];    // block scales
};

__device__ __forceinline__ float4 load_q4(const float* __restrict__ rows, int n_rows) {
    const int t = threadIdx.x;
    if ((t >> 5) >= n_rows || t >= 32 * kMaxRows) return make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    return *reinterpret_cast<const float4*>(rows + (size_t)(t >> 5) * kHD + 4 * (t & 31));
}

__device__ __forceinline__ void quantize_q4(float4 x, int n_rows, QSmem& sm) {
#pragma clang fp contract(off)
    const int t = threadIdx.x;
    const int H = t >> 5;
    if (H < n_rows && H < kMaxRows) {
        float mx = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
        mx = fmaxf(mx, dpp_f<kDppXor1>(mx));
        mx = fmaxf(mx, dpp_f<kDppXor2>(mx));
        mx = fmaxf(mx, dpp_f<kDppHalfMirror>(mx));
        if (mx < 1e-6f) mx = 1.0f;
        constexpr float kInv127 = 1.0f / 127.0f;
        const float qsc = mx * kInv127;
        const float iq = 127.0f / mx;
        const float xs[4] = {x.x, x.y, x.z, x.w};
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float r = roundf(xs[e] * iq);
            r = fminf(fmaxf(r, -128.0f), 127.0f);
            w |= ((uint32_t)(int)r & 0xFFu) << (8 * e);
        }
        sm.qc[H][t & 31] = w;
        if ((t & 7) == 0) sm.qs[H][(t & 31) >> 3] = qsc;
    }
}

// LDS-only barrier: waits for this wave's LDS traffic (not for its loads in
// flight), then for the workgroup.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Rounding a quotient to an integer without dividing (the decode's fused
// write path; the other write paths use an FMA onto a fixed-point grid).  The
// quantizer rounds x / d, the IEEE quotient, to nearest.  q = x * rcp(d), with
// v_rcp_f32 within one ulp of 1 / d, lies within |q| * 2^-21 of that quotient
// for normal operands, so rounding q gives the same integer unless one of the
// two lies within that distance of a half-integer.  For |q| <= 128,
// `near_half_small` flags q within 2^-11 of one (`rq` is rintf(q); a q that is
// not finite is flagged too); there the caller divides.
__device__ __forceinline__ bool near_half_small(float q, float rq) {
    return !(fabsf(q - rq) <= 0.5f - 0x1p-11f);
}

// Division by the kv-head count without the integer-divide sequence: for
// 0 <= t < 2^31 and n >= 1, m = ceil(2^(32+s) / n) with 2^s >= n gives
// t / n = (t * m) >> (32 + s) exactly.  m exceeds 2^(32+s) / n by less than
// one, so t * m / 2^(32+s) exceeds t / n by less than t / 2^(32+s) <
// 2^(-1-s) < 1 / n, which keeps it below the next integer.  Built on the host.
struct DivN {
    uint64_t m;
    int shift;
    int n;
};

inline DivN make_divn(int n) {
    int s = 0;
    while ((1LL << s) < n) ++s;
    return DivN{((1ULL << (32 + s)) + (uint64_t)n - 1) / (uint64_t)n, 32 + s, n};
}

__device__ __forceinline__ int div_n(int t, const DivN& d) {
    return (int)(((uint64_t)(uint32_t)t * d.m) >> d.shift);
}

// Storage order of the int8 pool's code rows.  The codes of a token slot s
// form one row of nkv x 128 bytes; head kh of that slot sits at column
//   (kh & ~(P - 1)) | ((kh + s) & (P - 1)),
// P = the largest power of two dividing nkv, at most 8: within each aligned
// group of P heads the heads rotate with the slot (P = 1 keeps column kh).
// A kv-head's rows then spread over every column position of the row
// instead of one: reading one fixed 128-byte column of many 1 KB rows is
// slower for some positions than for others on this memory system, and
// the decode's work items each read one head.  P divides the block size
// and a tile's token groups start on block boundaries, so the column of a
// load depends only on the lane.  The steps are not rotated.
__host__ __device__ __forceinline__ int q8_rot_group(int nkv) {
    const int p = nkv & -nkv;
    return p < 8 ? p : 8;
}
__host__ __device__ __forceinline__ int q8_col(int kh, long slot, int p) {
    return (kh & ~(p - 1)) | ((kh + (int)(slot & 7)) & (p - 1));
}

// Row order of the int4 and 2-bit pools (codes, scales and zeros alike):
// head-major inside each block, row ((slot / kv_bs) * nkv + kh) * kv_bs +
// slot % kv_bs, so the kv_bs rows of one (block, kv-head) are contiguous
// (1 KB of int4 codes for 16 slots) and a decode work item, which reads one
// kv-head, reads whole cache lines.
__host__ __device__ __forceinline__ size_t hm_row(long slot, int kh, int nkv, int log2_bs) {
    return ((((size_t)slot >> log2_bs) * (size_t)nkv + (size_t)kh) << log2_bs) |
           ((size_t)slot & (((size_t)1 << log2_bs) - 1));
}
__device__ __forceinline__ uint32_t hm_row32(uint32_t slot, uint32_t kh, uint32_t nkv, int log2_bs) {
    return (((slot >> log2_bs) * nkv + kh) << log2_bs) | (slot & ((1u << log2_bs) - 1));
}

// Storage order of an int4 key row (64 bytes, two codes per byte, even element
// in the high nibble): eight 8-byte parts, part 2c + h holding the pairs 32h +
// 8c .. 32h + 8c + 7, i.e. codes 64h + 16c .. 64h + 16c + 15, so that the 16
// bytes at 16c carry the same 16 d of both code groups (one 16-byte load per
// decode lane).  The byte offset of pairs 4w .. 4w + 3 (w = 0..15):
__host__ __device__ __forceinline__ unsigned q4_key_offset(int w) {
    return 16u * (unsigned)((w >> 1) & 3) + 8u * (unsigned)(w >> 3) + 4u * (unsigned)(w & 1);
}

// IEEE binary16 bits (low 16 bits of v) widened to float (exact)
__device__ __forceinline__ float half_bits_f(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)v);
}

// A lane's 16 consecutive input values of a write path as loaded (16
// float32 or 16 binary16 / bfloat16 values), and widened to float (exact).
template <int DT>
struct Raw16 {
    uint4 u[DT == KVQ8_F32 ? 4 : 2];
};

template <int DT>
__device__ __forceinline__ void load_raw16(const void* base, size_t byte_off, Raw16<DT>& r) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const char*>(base) + byte_off);
#pragma unroll
    for (int i = 0; i < (DT == KVQ8_F32 ? 4 : 2); ++i) r.u[i] = p[i];
}

template <int DT>
__device__ __forceinline__ void unpack_raw16(const Raw16<DT>& r, float (&x)[16]) {
#pragma unroll
    for (int i = 0; i < (DT == KVQ8_F32 ? 4 : 2); ++i) {
        const uint32_t w[4] = {r.u[i].x, r.u[i].y, r.u[i].z, r.u[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (DT == KVQ8_F32) {
                x[4 * i + j] = __uint_as_float(w[j]);
            } else if constexpr (DT == KVQ8_BF16) {
                x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
                x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            } else {
                x[8 * i + 2 * j] = half_bits_f(w[j] & 0xFFFFu);
                x[8 * i + 2 * j + 1] = half_bits_f(w[j] >> 16);
            }
        }
    }
}


// The [P4] Sec. 3.2 group quantizer at QMAX = 2^bits - 1 for a 64-value group
// held by a quad, 16 values per lane: scale = (max - min) / QMAX (1 for a
// constant group), floored at 1e-7 and rounded to binary16 (s16) before use;
// zero = rint(-min / s) clamped to [0, QMAX] (z16 its binary16 bits, +0.0 for
// zero).  Returns the lane's codes, byte i of b[h] the code of value 4h + i.
//
// code = clamp(rint(x / s + z), 0, QMAX), z an integer.  f = fma(x, rcp(s),
// z + 128.5 + 2^-15), clamped to [128.25, 128.75 + QMAX], lies in [128,
// 256): its unit is 2^-16 and its mantissa is (x * rcp(s) + z + 0.5) * 2^16,
// rounded, plus 2, so bits 16..19 are the code and bits 0..15 the fraction
// plus 2.  The clamp holds x / s + z below -0.25 at code 0 and above QMAX +
// 0.25 at QMAX, where every rounding gives that code.  Where the low bits are
// 0..3 the quotient + z lies within 2^-15 of a half-integer and the lane
// divides instead; elsewhere it lies at least 1.5 * 2^-16 from one, more than
// one rcp error (|x / s| <= 16: 2^-19) plus the division's and the
// addition's roundings (2^-19 each), so the code read from f is the correctly
// rounded rint's.
template <int QMAX>
__device__ __forceinline__ void quad_group_codes(const float (&x)[16], uint32_t (&b)[4], uint16_t& s16,
                                                 uint16_t& z16) {
#pragma clang fp contract(off)
    float mx = x[0], mn = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) {
        mx = fmaxf(mx, x[e]);
        mn = fminf(mn, x[e]);
    }
    mx = fmaxf(mx, dpp_f<kDppXor1>(mx));
    mn = fminf(mn, dpp_f<kDppXor1>(mn));
    mx = fmaxf(mx, dpp_f<kDppXor2>(mx));
    mn = fminf(mn, dpp_f<kDppXor2>(mn));
    float s32 = (mx == mn) ? 1.0f : (mx - mn) / (float)QMAX;
    s32 = fmaxf(s32, 1e-7f);
    s16 = __builtin_bit_cast(uint16_t, (_Float16)s32);
    const float s = half_bits_f(s16);
    // + 0.0f stores a zero as +0.0
    const float z = fminf(fmaxf(rintf(-mn / s), 0.0f), (float)QMAX) + 0.0f;
    z16 = __builtin_bit_cast(uint16_t, (_Float16)z);
    const float rs = __builtin_amdgcn_rcpf(s);
    const float m = z + 128.500030517578125f;       // exact: z is an integer
    uint32_t cb[16];                                 // bits 16..19: the code
    uint64_t slow[16];                               // wave masks of the lanes that divide
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        cb[e] = __float_as_uint(__builtin_amdgcn_fmed3f(__builtin_fmaf(x[e], rs, m), 128.25f, 128.75f + QMAX));
        slow[e] = __builtin_amdgcn_ballot_w64((uint16_t)cb[e] <= 3u);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (slow[e] != 0) {                         // rare: one wave-uniform test per value
            const float cd = fminf(fmaxf(rintf(x[e] / s + z), 0.0f), (float)QMAX);
            cb[e] = ((slow[e] >> (threadIdx.x & 63)) & 1) ? (uint32_t)(int)cd << 16 : cb[e];
        }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h)
        b[h] = __builtin_amdgcn_perm(cb[4 * h + 1], cb[4 * h], 0x0C0C0602u) |
               __builtin_amdgcn_perm(cb[4 * h + 3], cb[4 * h + 2], 0x06020C0Cu);
}

// The lanes of a row in the int4 and 2-bit write kernels (one (token,
// kv-head, K-or-V) row per 8 lanes, rows alternating K and V): lane l of the
// 8-lane group holds elements 64g + 16c .. 64g + 16c + 15 with g = l / 4 and
// c = l % 4 for g = 0, 3 - l % 4 for g = 1.  Each 64-value group is a quad,
// and lanes l and 7 - l (one half-mirror DPP step) hold the same c of the
// two groups.
struct GroupLane {
    int g, c, kind;
    __device__ __forceinline__ GroupLane() {
        const int l8 = threadIdx.x & 7;
        g = l8 >> 2;
        c = g ? 3 - (l8 & 3) : (l8 & 3);
        kind = (threadIdx.x >> 3) & 1;             // rows alternate K, V (groups 32 apart are even)
    }
};

// Pair q of the write kernels' n pairs per kv-head, taken kv-head-major
// (q = kv-head * n + i), so consecutive rows are consecutive tokens of one
// kv-head: contiguous rows of a head-major pool when their slots are.
__device__ __forceinline__ void head_major_pair(int q, const DivN& n, int& i, int& kh) {
    kh = div_n(q, n);
    i = q - kh * n.n;
}

}  // namespace kvq
