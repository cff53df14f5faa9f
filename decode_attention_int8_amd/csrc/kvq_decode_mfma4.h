// Mixed int4 / int8 cache on the matrix cores ([P4] Sec. 3.2-3.3 codes, the
// [P3] Sec. 2 single pass): chunks of the int4 pool and of the int8 window
// pool share one launch and one merge; int8 chunks run the int8 tile code.
//
// int4 tile (64 tokens, lane = (g, m) as in the int8 kernel), up to 8 query
// heads in one operand set:
//
// Q.K: v_mfma_i32_16x16x64_i8 per (token group v, code group h).  A = unsigned
//   codes of token 16v+m, d = 64h+16g .. +15, unpacked from 8 packed bytes as
//   [even d | odd d] per 4-byte word (two VALU ops per word); the key row's
//   storage order (q4_key_offset) puts both groups' bytes of lane group g in
//   one 16-byte load.  B = the query
//   codes in the same order, column c = (head c/2, block parity c%2):
//   column c receives P_b = sum q*c over block 2h + (c & 1), which lies in
//   code group h.  The score term of a block is qsc_b * s_h * (P_b - z_h R_b)
//   with R_b = sum q over the block (exact integers, applied in float).
//
// P.V: v_mfma_f32_16x16x32_f16 per (pair of token groups, d-slice s).  A
//   value row stores the pair 64G + 4m + 2k, +1 at byte 4m + 2G + k, so the
//   word of lane m holds d = 4m .. 4m+3 of both code groups and slice s
//   covers d = 64(s/4) + 4m + (s%4): group s/4 for every column.  Its A
//   operand is the weights p * vscale of that group (f16 high part or
//   remainder below it, times 2^E; row c = (head c/2, part c%2)) and B is
//   the code c as f16.  A byte holding a code 0..15 is, read as an OCP fp8
//   e4m3 number, exactly c * 2^-9, so one fp8 -> f16 conversion with scale
//   2^9 turns two tokens' code bytes into the exact f16 pair.  The zero
//   points enter through one more product per group and token pair, with B
//   = z of each token in every column: sum_t w_t z_t, subtracted from every
//   slice of the group when the wave folds its state (sum w (c - z) = sum w c
//   - sum w z, both exact integers times the same weights).  Each lane's
//   softmax values are exactly the weights it supplies.
#pragma once

#include "kvq_decode_mfma_kernel.h"

namespace kvq {

// LDS of the mixed kernel: the int8 layout plus per-token int4 scales.
struct MSmem4 : MSmem {
    float k4s[kWaves][2][64];      // key group scale * score scale (0 if masked)
    float k4z[kWaves][2][64];      // key group zero point
    float v4s[kWaves][2][64];      // value group scale * 2^E (0 if masked)
    uint16_t v4z[kWaves][2][64];   // binary16 value zero point (0 if masked)
};

// Wave state of the group walks: the int8 walk's plus, per code group, the
// products of the weights with the value zero points (same rows as acc, the
// same value in every column).
struct MStateG : MState {
    v4f_t accz[2];
};

// two code bytes (word half HI) -> their values as an f16 pair: a byte
// 0..15 is c * 2^-9 as fp8 e4m3, scaled by 2^9
template <bool HI>
__device__ __forceinline__ uint32_t fp8_codes_f16x2(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 512.0f, HI));
}

struct MTile4 {
    v2u_t k[4][2];       // [v][h]: token 16v+m, codes 64h + 16g .. +15 (row bytes 16g + 8h .. +7)
    uint32_t v[4][4];    // [v][e]: token 16v+4g+e, packed bytes 4m .. 4m+3
    uint32_t ks, kz, vs, vz;   // token base+lane: both groups' binary16 scale / zero
    int id;
};

struct MQuery4 {
    v4i_t op[2];         // [h] B operand (codes in [even | odd] order)
    float sc[2];         // [h] query block scale of column m
    float R[2];          // [h] sum of the query codes of that block
};

// codes of 16 consecutive d (4 words, natural order) -> [even | odd] per 8
__device__ __forceinline__ v4i_t even_odd_order(v4u_t n) {
    return v4i_t{(int)__builtin_amdgcn_perm(n.y, n.x, 0x06040200u), (int)__builtin_amdgcn_perm(n.y, n.x, 0x07050301u),
                 (int)__builtin_amdgcn_perm(n.w, n.z, 0x06040200u), (int)__builtin_amdgcn_perm(n.w, n.z, 0x07050301u)};
}

// 8 packed bytes (16 codes, even d in the high nibbles) -> 16 code bytes in
// [even | odd] order per 4-byte word
__device__ __forceinline__ v4i_t unpack_q4(v2u_t w) {
    return v4i_t{(int)((w.x >> 4) & kNib), (int)(w.x & kNib), (int)((w.y >> 4) & kNib), (int)(w.y & kNib)};
}

// The query operand of the group tiles; EVEN_ODD orders each word's codes as
// the int4 key unpacking does, otherwise they stay in natural order (2-bit
// keys).
template <bool EVEN_ODD = true>
__device__ __forceinline__ MQuery4 load_q4_operand(const QSmem& sm, int G, int g, int m) {
    MQuery4 Q;
    const int H = m >> 1;
    const bool live = H < G;
    const int Hc = live ? H : 0;
    const bool mine = live && ((g >> 1) == (m & 1));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const v4u_t c = *reinterpret_cast<const v4u_t*>(&sm.qc[Hc][16 * h + 4 * g]);
        if constexpr (EVEN_ODD)
            Q.op[h] = mine ? even_odd_order(c) : v4i_t{0, 0, 0, 0};
        else
            Q.op[h] = mine ? __builtin_bit_cast(v4i_t, c) : v4i_t{0, 0, 0, 0};
        const int blk = 2 * h + (m & 1);
        Q.sc[h] = live ? sm.qs[Hc][blk] : 0.0f;
        int r = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) r = __builtin_amdgcn_sdot4((int)sm.qc[Hc][8 * blk + i], 0x01010101, r, false);
        Q.R[h] = live ? (float)r : 0.0f;
    }
    return Q;
}

struct LaneOff4 {
    uint32_t k;          // packed key row of token 16v+m, bytes 16g .. 16g+15 (q4_key_offset order)
    uint32_t v[4];       // packed value rows of tokens 16v+4g+e, bytes 4m..
};

__device__ __forceinline__ LaneOff4 lane_offsets4(const DecodeArgs& a, int lane) {
    const int g = lane >> 4;
    const int m = lane & 15;
    (void)a;
    LaneOff4 o;
    o.k = (uint32_t)m * (kHD / 2) + 16 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) o.v[e] = (uint32_t)(4 * g + e) * (kHD / 2) + 4 * m;
    return o;
}

// Issue all loads of an int4 tile (rows of invalid blocks read slot 0).
template <bool BS8>
__device__ __forceinline__ void mtile4_issue(const DecodeArgs& a, int raw, int base, int kh, int lane,
                                             const LaneOff4& lo, MTile4& T) {
    const int g = lane >> 4;
    const int m = lane & 15;
    const uint32_t bs_mask = (1u << a.log2_bs) - 1;
    const int id = (raw >= 0 && raw < a.r4.n_blocks) ? raw : -1;
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
            const uint8_t* pk = a.k4 + (size_t)u * (kHD / 2);
            const uint8_t* pv = a.v4 + (size_t)u * (kHD / 2);
            const v4u_t kk = *reinterpret_cast<const v4u_t*>(pk + lo.k);
            T.k[v][0] = v2u_t{kk.x, kk.y};
            T.k[v][1] = v2u_t{kk.z, kk.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) T.v[v][e] = *reinterpret_cast<const uint32_t*>(pv + lo.v[e]);
        } else {
            const uint32_t u0 = grp(2 * v), u1 = grp(2 * v + 1);
            const uint32_t rk = ((m & 8) ? u1 : u0) + (uint32_t)(m & 7);
            const v4u_t kk = *reinterpret_cast<const v4u_t*>(a.k4 + (size_t)rk * (kHD / 2) + 16 * g);
            T.k[v][0] = v2u_t{kk.x, kk.y};
            T.k[v][1] = v2u_t{kk.z, kk.w};
            const uint32_t rv = ((g & 2) ? u1 : u0) + (uint32_t)(4 * (g & 1));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                T.v[v][e] = *reinterpret_cast<const uint32_t*>(a.v4 + (size_t)(rv + (uint32_t)e) * (kHD / 2) + 4 * m);
        }
    }
    const uint32_t srow = id >= 0 ? ((((uint32_t)id * nkv + kh) << a.log2_bs) + (((uint32_t)base + lane) & bs_mask)) : 0u;
    T.ks = *reinterpret_cast<const uint32_t*>(a.k4s + (size_t)srow * 2);
    T.kz = *reinterpret_cast<const uint32_t*>(a.k4z + (size_t)srow * 2);
    T.vs = *reinterpret_cast<const uint32_t*>(a.v4s + (size_t)srow * 2);
    T.vz = *reinterpret_cast<const uint32_t*>(a.v4z + (size_t)srow * 2);
}

__device__ __forceinline__ void mtile4_compute(const DecodeArgs& a, const MTile4& T, int base, int L, int lane,
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
#pragma unroll
        for (int h = 0; h < 2; ++h)
            P[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack_q4(T.k[v][h]), Q.op[h], v4i_t{0, 0, 0, 0}, 0, 0, 0);
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
        // accumulator rows of this lane: heads 2g and 2g+1, whose factors sit
        // in lanes 4g and 4g+2
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
        // codes of slice sl (d = 64(sl/4) + 4m + sl%4: byte sl/2 of the word,
        // high nibble for even sl) for tokens 2i, 2i+1 of the lane's 8
        // (token group 2vp + q/4, e = q%4) as one f16 pair
        uint32_t bw[8][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q0 = 2 * i, q1 = 2 * i + 1;
            const uint32_t wa = T.v[2 * vp + q0 / 4][q0 % 4], wb = T.v[2 * vp + q1 / 4][q1 % 4];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                // bytes [a(2hb), b(2hb), a(2hb+1), b(2hb+1)]
                const uint32_t x = __builtin_amdgcn_perm(wb, wa, hb ? 0x07030602u : 0x05010400u);
                const uint32_t xh = (x >> 4) & kNib, xl = x & kNib;
                bw[4 * hb + 0][i] = fp8_codes_f16x2<false>(xh);
                bw[4 * hb + 1][i] = fp8_codes_f16x2<false>(xl);
                bw[4 * hb + 2][i] = fp8_codes_f16x2<true>(xh);
                bw[4 * hb + 3][i] = fp8_codes_f16x2<true>(xl);
            }
        }
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            const v8h_t B = __builtin_bit_cast(v8h_t, v4u_t{bw[sl][0], bw[sl][1], bw[sl][2], bw[sl][3]});
            st.acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[sl >> 2], B, st.acc[sl], 0, 0, 0);
        }
    }
}

// Fold a group-walk wave state into the workgroup's LDS layout (per wave and
// head: M, S, acc[128]); slice s of lane m holds d = 64(s/4) + 4m + s%4, and
// the zero-point products of its group come off here.
__device__ __forceinline__ void mwave4_to_lds(MSmem4& sm, MStateG& st, int G, int lane, int wave) {
    const int g = lane >> 4;
    const int m = lane & 15;
    float S = st.S;
    S += swz_xor16(S);
    S += xor32(S);
    if (g == 0 && (m & 1) == 0 && (m >> 1) < G) {
        sm.m[wave][m >> 1] = st.M;
        sm.s[wave][m >> 1] = S;
    }
    const float unscale = exp2i(-st.E);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int H = 2 * g + hh;
        if (H < G) {
            float o[8];
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                const v4f_t& z = st.accz[sl >> 2];
                o[sl] = ((st.acc[sl][2 * hh] - z[2 * hh]) + (st.acc[sl][2 * hh + 1] - z[2 * hh + 1])) * unscale;
            }
            *reinterpret_cast<float4*>(&sm.acc[wave][H][4 * m]) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(&sm.acc[wave][H][64 + 4 * m]) = make_float4(o[4], o[5], o[6], o[7]);
        }
    }
}

}  // namespace kvq
