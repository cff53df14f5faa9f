// 2-bit band of the group variant on the matrix cores ([P4] Sec. 3.2 group
// codes at two bits, Sec. 3.3 bands; the [P3] Sec. 2 single pass): the int4
// tile's operand scheme with four codes per byte.
//
// Q.K: v_mfma_i32_16x16x64_i8 per (token group v, row half h).  Key word
//   2g + h of token 16v+m holds d = 64h + 16g + 4k + j at bits 8j + 2k, so
//   (word >> 2k) & 0x03030303 is the k-th 4-byte part of the A operand with
//   the codes in natural order; B = the query codes in natural order, column
//   c = (head c/2, block parity).  The score term is the int4 tile's,
//   qsc_b * s_h * (P_b - z_h R_b).
//
// P.V: the 16-bit word m of a value row holds d = 64(s/4) + 4m + s%4 at bits
//   2s, the int4 tile's slice order.  Two tokens' words interleaved byte by
//   byte give, after a shift by 2(s%4) and a mask, both tokens' codes of
//   slices s and s + 4 as four bytes; two fp8 -> f16 conversions (as in the
//   int4 tile) make them the exact f16 pairs of both slices.  The weights (A
//   operand, one per code group) and the zero-point products are the int4
//   tile's.
#pragma once

#include "kvq_decode_mfma4.h"

namespace kvq {

constexpr int kRow2 = kHD / 4;     // bytes of a 2-bit row
constexpr uint32_t kCrumb = 0x03030303u;

struct MTile2 {
    v2u_t k[4];          // [v]: token 16v+m, key words 2g (h = 0) and 2g+1 (h = 1)
    uint32_t v[4][4];    // [v][e]: token 16v+4g+e, value bytes 2m, 2m+1 (low 16 bits)
    uint32_t ks, kz, vs, vz;   // token base+lane: both groups' binary16 scale / zero
    int id;
};

struct LaneOff2 {
    uint32_t k;          // key row of token 16v+m, bytes 8g..
    uint32_t v[4];       // value rows of tokens 16v+4g+e, bytes 2m..
};

__device__ __forceinline__ LaneOff2 lane_offsets2(const BandArgs& a, int lane) {
    const int g = lane >> 4;
    const int m = lane & 15;
    (void)a;
    LaneOff2 o;
    o.k = (uint32_t)m * kRow2 + 8 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) o.v[e] = (uint32_t)(4 * g + e) * kRow2 + 2 * m;
    return o;
}

// 4 packed bytes (16 codes of d = 16g' .. 16g'+15) -> 16 code bytes in
// natural order
__device__ __forceinline__ v4i_t unpack_q2(uint32_t w) {
    return v4i_t{(int)(w & kCrumb), (int)((w >> 2) & kCrumb), (int)((w >> 4) & kCrumb), (int)((w >> 6) & kCrumb)};
}

// Issue all loads of a 2-bit tile (rows of invalid blocks read slot 0).
template <bool BS8>
__device__ __forceinline__ void mtile2_issue(const BandArgs& a, int raw, int base, int kh, int lane,
                                             const LaneOff2& lo, MTile2& T) {
    const int g = lane >> 4;
    const int m = lane & 15;
    const uint32_t bs_mask = (1u << a.log2_bs) - 1;
    const int id = (raw >= 0 && raw < a.r2.n_blocks) ? raw : -1;
    T.id = id;
    const uint32_t nkv = (uint32_t)a.nkv;
    auto grp = [&](int i) __attribute__((always_inline)) -> uint32_t {
        const int idi = __builtin_amdgcn_readlane(id, 8 * i);
        // a block outside the pool reads block 0 (in bounds; its tokens are masked)
        const uint32_t idc = (uint32_t)max(idi, 0);
        return ((idc * nkv + kh) << a.log2_bs) + (((uint32_t)base + 8 * i) & bs_mask);
    };
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        if constexpr (!BS8) {
            const uint32_t u = grp(2 * v);
            T.k[v] = *reinterpret_cast<const v2u_t*>(a.k2 + (size_t)u * kRow2 + lo.k);
            const uint8_t* pv = a.v2 + (size_t)u * kRow2;
#pragma unroll
            for (int e = 0; e < 4; ++e) T.v[v][e] = *reinterpret_cast<const uint16_t*>(pv + lo.v[e]);
        } else {
            const uint32_t u0 = grp(2 * v), u1 = grp(2 * v + 1);
            const uint32_t rk = ((m & 8) ? u1 : u0) + (uint32_t)(m & 7);
            T.k[v] = *reinterpret_cast<const v2u_t*>(a.k2 + (size_t)rk * kRow2 + 8 * g);
            const uint32_t rv = ((g & 2) ? u1 : u0) + (uint32_t)(4 * (g & 1));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                T.v[v][e] = *reinterpret_cast<const uint16_t*>(a.v2 + (size_t)(rv + (uint32_t)e) * kRow2 + 2 * m);
        }
    }
    const uint32_t srow = id >= 0 ? ((((uint32_t)id * nkv + kh) << a.log2_bs) + (((uint32_t)base + lane) & bs_mask)) : 0u;
    T.ks = *reinterpret_cast<const uint32_t*>(a.k2s + (size_t)srow * 2);
    T.kz = *reinterpret_cast<const uint32_t*>(a.k2z + (size_t)srow * 2);
    T.vs = *reinterpret_cast<const uint32_t*>(a.v2s + (size_t)srow * 2);
    T.vz = *reinterpret_cast<const uint32_t*>(a.v2z + (size_t)srow * 2);
}

__device__ __forceinline__ void mtile2_compute(const BandArgs& a, const MTile2& T, int base, int L, int lane,
                                               int wave, const MQuery4& Q, MStateG& st, MSmem4& sm) {
    const int g = lane >> 4;
    const int m = lane & 15;
    // per-token scales through LDS (lane l holds token base+l)
    {
        const bool ok = (base + lane < L) && T.id >= 0;
        const float vs0 = half_bits_f(T.vs & 0xFFFFu), vs1 = half_bits_f(T.vs >> 16);
        const float vm = __int_as_float(
            __builtin_amdgcn_readfirstlane(__float_as_int(wave_max(ok ? fmaxf(vs0, vs1) : 0.0f))));
        if (vm > 0.0f) {
            const int e = (int)((__float_as_uint(vm) >> 23) & 0xFFu) - 127;
            const int Et = min(max(14 - e, -100), 100);
            if (Et < st.E) {
                const float f = exp2i(Et - st.E);
#pragma unroll
                for (int sl = 0; sl < 8; ++sl) st.acc[sl] *= f;
                st.accz[0] *= f;
                st.accz[1] *= f;
                st.E = Et;
            }
        }
        const float sc = exp2i(st.E);
        sm.k4s[wave][0][lane] = ok ? half_bits_f(T.ks & 0xFFFFu) * a.score_scale : 0.0f;
        sm.k4s[wave][1][lane] = ok ? half_bits_f(T.ks >> 16) * a.score_scale : 0.0f;
        sm.k4z[wave][0][lane] = ok ? half_bits_f(T.kz & 0xFFFFu) : 0.0f;
        sm.k4z[wave][1][lane] = ok ? half_bits_f(T.kz >> 16) : 0.0f;
        sm.kb[wave][lane] = ok ? 0.0f : -INFINITY;
        sm.v4s[wave][0][lane] = ok ? vs0 * sc : 0.0f;
        sm.v4s[wave][1][lane] = ok ? vs1 * sc : 0.0f;
        sm.v4z[wave][0][lane] = ok ? (uint16_t)(T.vz & 0xFFFFu) : (uint16_t)0;
        sm.v4z[wave][1][lane] = ok ? (uint16_t)(T.vz >> 16) : (uint16_t)0;
    }
    // Q.K and scores
    float s[4][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        v4i_t P[2];
        P[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack_q2(T.k[v].x), Q.op[0], v4i_t{0, 0, 0, 0}, 0, 0, 0);
        P[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack_q2(T.k[v].y), Q.op[1], v4i_t{0, 0, 0, 0}, 0, 0, 0);
        const float4 ks0 = *reinterpret_cast<const float4*>(&sm.k4s[wave][0][16 * v + 4 * g]);
        const float4 ks1 = *reinterpret_cast<const float4*>(&sm.k4s[wave][1][16 * v + 4 * g]);
        const float4 kz0 = *reinterpret_cast<const float4*>(&sm.k4z[wave][0][16 * v + 4 * g]);
        const float4 kz1 = *reinterpret_cast<const float4*>(&sm.k4z[wave][1][16 * v + 4 * g]);
        const float4 kb = *reinterpret_cast<const float4*>(&sm.kb[wave][16 * v + 4 * g]);
        const float kS[2][4] = {{ks0.x, ks0.y, ks0.z, ks0.w}, {ks1.x, ks1.y, ks1.z, ks1.w}};
        const float kZ[2][4] = {{kz0.x, kz0.y, kz0.z, kz0.w}, {kz1.x, kz1.y, kz1.z, kz1.w}};
        const float kB[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // P - z R is an exact integer below 2^17 in float
            float f = fmaf(-kZ[0][r], Q.R[0], (float)P[0][r]) * (Q.sc[0] * kS[0][r]);
            f = fmaf(fmaf(-kZ[1][r], Q.R[1], (float)P[1][r]), Q.sc[1] * kS[1][r], f);
            s[v][r] = f + dpp_f<kDppXor1>(f) + kB[r];
        }
    }
    // softmax: lane (g, m) owns head m/2 for tokens 16v + 4g + r
    float mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[v][r]);
    mt = fmaxf(mt, swz_xor16(mt));
    mt = fmaxf(mt, xor32(mt));
    if (__builtin_amdgcn_ballot_w64(mt > st.M) != 0) {
        const float fac = (mt > st.M) ? __builtin_amdgcn_exp2f(st.M - mt) : 1.0f;
        st.M = fmaxf(st.M, mt);
        st.S *= fac;
        const float fa = bperm_f(fac, 4 * g);
        const float fb = bperm_f(fac, 4 * g + 2);
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            st.acc[sl][0] *= fa;
            st.acc[sl][1] *= fa;
            st.acc[sl][2] *= fb;
            st.acc[sl][3] *= fb;
        }
#pragma unroll
        for (int G2 = 0; G2 < 2; ++G2) {
            st.accz[G2][0] *= fa;
            st.accz[G2][1] *= fa;
            st.accz[G2][2] *= fb;
            st.accz[G2][3] *= fb;
        }
    }
    const float mref = (st.M == -INFINITY) ? 0.0f : st.M;
    const uint32_t part_mask = weight_part_mask(m);
    float p[4][4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[v][r] = __builtin_amdgcn_exp2f(s[v][r] - mref);
            st.S += p[v][r];
        }
    // P.V: one A operand per code group, the codes as f16, the zero points
    // through their own product per group
#pragma unroll
    for (int vp = 0; vp < 2; ++vp) {
        v8h_t A[2];
        uint32_t zc[2][4];      // [group]: binary16 z of the lane's 8 tokens, in pairs
#pragma unroll
        for (int G2 = 0; G2 < 2; ++G2) {
            uint32_t wop[2][2];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int v = 2 * vp + q2;
                const float4 vv = *reinterpret_cast<const float4*>(&sm.v4s[wave][G2][16 * v + 4 * g]);
                const float w[4] = {p[v][0] * vv.x, p[v][1] * vv.y, p[v][2] * vv.z, p[v][3] * vv.w};
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    wop[q2][pr] = weight_part_f16x2(w[2 * pr], w[2 * pr + 1], part_mask);
                }
                const uint2 zz = *reinterpret_cast<const uint2*>(&sm.v4z[wave][G2][16 * v + 4 * g]);
                zc[G2][2 * q2] = zz.x;
                zc[G2][2 * q2 + 1] = zz.y;
            }
            A[G2] = __builtin_bit_cast(v8h_t, v4u_t{wop[0][0], wop[0][1], wop[1][0], wop[1][1]});
            const v8h_t Z = __builtin_bit_cast(v8h_t, v4u_t{zc[G2][0], zc[G2][1], zc[G2][2], zc[G2][3]});
            st.accz[G2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[G2], Z, st.accz[G2], 0, 0, 0);
        }
        // tokens 2i and 2i+1 of the lane's 8 (token group 2vp + q/4, e = q%4)
        // interleaved: bytes [a0, b0, a1, b1] of their 16-bit words, so slice
        // sl < 4 sits at bits 2sl of bytes 0-1 and slice sl + 4 of bytes 2-3
        uint32_t bw[8][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q0 = 2 * i, q1 = 2 * i + 1;
            const uint32_t tw = __builtin_amdgcn_perm(T.v[2 * vp + q1 / 4][q1 % 4], T.v[2 * vp + q0 / 4][q0 % 4],
                                                      0x05010400u);
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) {
                const uint32_t x = (tw >> (2 * sl)) & kCrumb;
                bw[sl][i] = fp8_codes_f16x2<false>(x);
                bw[sl + 4][i] = fp8_codes_f16x2<true>(x);
            }
        }
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            const v8h_t B = __builtin_bit_cast(v8h_t, v4u_t{bw[sl][0], bw[sl][1], bw[sl][2], bw[sl][3]});
            st.acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[sl >> 2], B, st.acc[sl], 0, 0, 0);
        }
    }
}

}  // namespace kvq
