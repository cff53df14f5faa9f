// Mixed int4 / int8 cache on the matrix cores ([P4] Sec. 3.2-3.3 codes, the
// [P3] Sec. 2 single pass): chunks of the int4 pool and of the int8 window
// pool share one launch and one merge; int8 chunks run the int8 tile code.
//
// int4 tile (64 tokens, lane = (g, m) as in the int8 kernel), query heads in
// sets of four (S = 0, 1):
//
// Q.K: v_mfma_i32_16x16x64_i8 per (token group v, row half h).  A = unsigned
//   codes of token 16v+m, d = 64h+16g .. +15, unpacked from 8 packed bytes as
//   [even d | odd d] per 4-byte word (two VALU ops per word); B = the query
//   codes in the same order, column c = (head 4S + c/4, block parity c%2):
//   column c receives P_b = sum q*c over block 2h + (c & 1).  The score term
//   of a block is qsc_b * s_g * (P_b - z_g * R_b) with R_b = sum q over the
//   block (exact integers, applied in float), g = h the code group.
//
// P.V: v_mfma_f32_16x16x32_f16 per (pair of token groups, d-slice s) and
//   head set.  The group scale differs between the two halves of a row, so
//   the weights carry it: row c = (head 4S + c/4, group (c/2)&1, part c&1),
//   A = p * vscale_{t,group} (f16 high part or rounded remainder, times 2^E);
//   B = c - z_{t,group of the column} as f16 (exact small integers), column
//   m <-> d = 8m + s, group m/8.  Rows whose group differs from the column's
//   are discarded; lane (g, m) keeps rows 2(m/8) and 2(m/8)+1 of head 4S+g.
//   Each lane's softmax values are exactly the weights it supplies.
#pragma once

#include "kvq_decode_mfma_kernel.h"

namespace kvq {

// LDS of the mixed kernel: the int8 layout plus per-token int4 scales.
struct MSmem4 : MSmem {
    float k4s[kWaves][2][64];      // key group scale * score scale (0 if masked)
    float k4z[kWaves][2][64];      // key group zero point
    float v4s[kWaves][2][64];      // value group scale * 2^E (0 if masked)
    uint16_t v4c[kWaves][2][64];   // binary16 of -(1024 + value zero point)
};

struct MTile4 {
    v2u_t k[4][2];       // [v][h]: token 16v+m, packed bytes 32h+8g .. +7
    uint32_t v[4][4];    // [v][e]: token 16v+4g+e, packed bytes 4m .. 4m+3
    uint32_t ks, kz, vs, vz;   // token base+lane: both groups' binary16 scale / zero
    int id;
};

struct MQuery4 {
    v4i_t op[2][2];      // [set][h] B operand (codes in [even | odd] order)
    float sc[2][2];      // [set][h] query block scale of column m
    float R[2][2];       // [set][h] sum of the query codes of that block
};

template <int NSET>
struct MState4 {
    float M[NSET];       // running max of head 4S + m/4
    float S[NSET];       // this lane's share of its sum
    int E;               // accumulator scale exponent (wave-uniform)
    v4f_t acc[NSET][8];  // [set][slice]: rows 4g+r (head 4S+g, group r/2, part r%2)
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

template <int NSET>
__device__ __forceinline__ MQuery4 load_q4_operand(const QSmem& sm, int G, int g, int m) {
    MQuery4 Q;
#pragma unroll
    for (int S = 0; S < NSET; ++S) {
        const int H = 4 * S + (m >> 2);
        const bool live = H < G;
        const int Hc = live ? H : 0;
        const bool mine = live && ((g >> 1) == (m & 1));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const v4u_t c = *reinterpret_cast<const v4u_t*>(&sm.qc[Hc][16 * h + 4 * g]);
            Q.op[S][h] = mine ? even_odd_order(c) : v4i_t{0, 0, 0, 0};
            const int blk = 2 * h + (m & 1);
            Q.sc[S][h] = live ? sm.qs[Hc][blk] : 0.0f;
            int r = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) r = __builtin_amdgcn_sdot4((int)sm.qc[Hc][8 * blk + i], 0x01010101, r, false);
            Q.R[S][h] = live ? (float)r : 0.0f;
        }
    }
    return Q;
}

struct LaneOff4 {
    uint32_t k;          // packed key row of token 16v+m, bytes 8g..
    uint32_t v[4];       // packed value rows of tokens 16v+4g+e, bytes 4m..
};

__device__ __forceinline__ LaneOff4 lane_offsets4(const DecodeArgs& a, int lane) {
    const int g = lane >> 4;
    const int m = lane & 15;
    const uint32_t row = (uint32_t)a.nkv * (kHD / 2);
    LaneOff4 o;
    o.k = (uint32_t)m * row + 8 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) o.v[e] = (uint32_t)(4 * g + e) * row + 4 * m;
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
        return idi >= 0 ? ((((uint32_t)idi << a.log2_bs) + (((uint32_t)base + 8 * i) & bs_mask)) * nkv + kh) : 0u;
    };
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        if constexpr (!BS8) {
            const uint32_t u = grp(2 * v);
            const uint8_t* pk = a.k4 + (size_t)u * (kHD / 2);
            const uint8_t* pv = a.v4 + (size_t)u * (kHD / 2);
            T.k[v][0] = *reinterpret_cast<const v2u_t*>(pk + lo.k);
            T.k[v][1] = *reinterpret_cast<const v2u_t*>(pk + lo.k + 32);
#pragma unroll
            for (int e = 0; e < 4; ++e) T.v[v][e] = *reinterpret_cast<const uint32_t*>(pv + lo.v[e]);
        } else {
            const uint32_t u0 = grp(2 * v), u1 = grp(2 * v + 1);
            const uint32_t rk = ((m & 8) ? u1 : u0) + (uint32_t)(m & 7) * nkv;
            const uint8_t* p = a.k4 + (size_t)rk * (kHD / 2) + 8 * g;
            T.k[v][0] = *reinterpret_cast<const v2u_t*>(p);
            T.k[v][1] = *reinterpret_cast<const v2u_t*>(p + 32);
            const uint32_t rv = ((g & 2) ? u1 : u0) + (uint32_t)(4 * (g & 1)) * nkv;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                T.v[v][e] = *reinterpret_cast<const uint32_t*>(a.v4 + (size_t)(rv + (uint32_t)e * nkv) * (kHD / 2) + 4 * m);
        }
    }
    const uint32_t srow = id >= 0 ? ((((uint32_t)id << a.log2_bs) + (((uint32_t)base + lane) & bs_mask)) * nkv + kh) : 0u;
    T.ks = *reinterpret_cast<const uint32_t*>(a.k4s + (size_t)srow * 2);
    T.kz = *reinterpret_cast<const uint32_t*>(a.k4z + (size_t)srow * 2);
    T.vs = *reinterpret_cast<const uint32_t*>(a.v4s + (size_t)srow * 2);
    T.vz = *reinterpret_cast<const uint32_t*>(a.v4z + (size_t)srow * 2);
}

template <int NSET>
__device__ __forceinline__ void mtile4_compute(const DecodeArgs& a, const MTile4& T, int base, int L, int lane,
                                               int wave, const MQuery4& Q, MState4<NSET>& st, MSmem4& sm) {
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
                for (int S = 0; S < NSET; ++S)
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl) st.acc[S][sl] *= f;
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
        // -(1024 + z) is exact in binary16 for z in [0, 15]
        const float z0 = ok ? half_bits_f(T.vz & 0xFFFFu) : 0.0f, z1 = ok ? half_bits_f(T.vz >> 16) : 0.0f;
        sm.v4c[wave][0][lane] = __builtin_bit_cast(uint16_t, (_Float16)(-(1024.0f + z0)));
        sm.v4c[wave][1][lane] = __builtin_bit_cast(uint16_t, (_Float16)(-(1024.0f + z1)));
    }
    // Q.K and scores
    float s[NSET][4][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        v4i_t P[NSET][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const v4i_t A = unpack_q4(T.k[v][h]);
#pragma unroll
            for (int S = 0; S < NSET; ++S)
                P[S][h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Q.op[S][h], v4i_t{0, 0, 0, 0}, 0, 0, 0);
        }
        const float4 ks0 = *reinterpret_cast<const float4*>(&sm.k4s[wave][0][16 * v + 4 * g]);
        const float4 ks1 = *reinterpret_cast<const float4*>(&sm.k4s[wave][1][16 * v + 4 * g]);
        const float4 kz0 = *reinterpret_cast<const float4*>(&sm.k4z[wave][0][16 * v + 4 * g]);
        const float4 kz1 = *reinterpret_cast<const float4*>(&sm.k4z[wave][1][16 * v + 4 * g]);
        const float4 kb = *reinterpret_cast<const float4*>(&sm.kb[wave][16 * v + 4 * g]);
        const float kS[2][4] = {{ks0.x, ks0.y, ks0.z, ks0.w}, {ks1.x, ks1.y, ks1.z, ks1.w}};
        const float kZ[2][4] = {{kz0.x, kz0.y, kz0.z, kz0.w}, {kz1.x, kz1.y, kz1.z, kz1.w}};
        const float kB[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
        for (int S = 0; S < NSET; ++S)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // P - z R is an exact integer below 2^17 in float
                float f = fmaf(-kZ[0][r], Q.R[S][0], (float)P[S][0][r]) * (Q.sc[S][0] * kS[0][r]);
                f = fmaf(fmaf(-kZ[1][r], Q.R[S][1], (float)P[S][1][r]), Q.sc[S][1] * kS[1][r], f);
                s[S][v][r] = f + dpp_f<kDppXor1>(f) + kB[r];
            }
    }
    // softmax per head set
    uint32_t wop[NSET][4][2];
    const int grp_row = (m >> 1) & 1;   // code group of this lane's weight row
    const bool lo_row = m & 1;
#pragma unroll
    for (int S = 0; S < NSET; ++S) {
        float mt = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[S][v][r]);
        mt = fmaxf(mt, swz_xor16(mt));
        mt = fmaxf(mt, xor32(mt));
        if (__builtin_amdgcn_ballot_w64(mt > st.M[S]) != 0) {
            const float fac = (mt > st.M[S]) ? __builtin_amdgcn_exp2f(st.M[S] - mt) : 1.0f;
            st.M[S] = fmaxf(st.M[S], mt);
            st.S[S] *= fac;
            // accumulator rows of this lane: head 4S + g, whose factor sits in lane 4g
            const float fa = bperm_f(fac, 4 * g);
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) st.acc[S][sl] *= fa;
        }
        const float mref = (st.M[S] == -INFINITY) ? 0.0f : st.M[S];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float4 vv = *reinterpret_cast<const float4*>(&sm.v4s[wave][grp_row][16 * v + 4 * g]);
            const float v4[4] = {vv.x, vv.y, vv.z, vv.w};
            float w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[S][v][r] - mref);
                st.S[S] += p;
                w[r] = p * v4[r];
            }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const float h0 = __uint_as_float(__float_as_uint(w[2 * pr]) & 0xFFFFE000u);
                const float h1 = __uint_as_float(__float_as_uint(w[2 * pr + 1]) & 0xFFFFE000u);
                const uint32_t hi = pack_f16_rtz(h0, h1);
                const uint32_t lo = pack_f16(w[2 * pr] - h0, w[2 * pr + 1] - h1);
                wop[S][v][pr] = lo_row ? lo : hi;
            }
        }
    }
    // P.V: value codes minus zero point as f16, shared by the head sets
    const int grp_col = m >> 3;
#pragma unroll
    for (int vp = 0; vp < 2; ++vp) {
        // -(1024 + z) for the 8 tokens of this lane's k-range, in pairs
        uint32_t zc[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint2 zz = *reinterpret_cast<const uint2*>(&sm.v4c[wave][grp_col][16 * (2 * vp + q) + 4 * g]);
            zc[2 * q] = zz.x;
            zc[2 * q + 1] = zz.y;
        }
        // even / odd codes of the 8 tokens' words
        uint32_t ev[8], od[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t w = T.v[2 * vp + q / 4][q % 4];
            ev[q] = (w >> 4) & kNib;
            od[q] = w & kNib;
        }
        v8h_t A[NSET];
#pragma unroll
        for (int S = 0; S < NSET; ++S)
            A[S] = __builtin_bit_cast(v8h_t, v4u_t{wop[S][2 * vp][0], wop[S][2 * vp][1], wop[S][2 * vp + 1][0],
                                                   wop[S][2 * vp + 1][1]});
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            // d = 8m + sl: byte sl/2 of the word, high nibble for even sl
            const int byte = sl >> 1;
            uint32_t bw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t xa = (sl & 1) ? od[2 * i] : ev[2 * i];
                const uint32_t xb = (sl & 1) ? od[2 * i + 1] : ev[2 * i + 1];
                // [code_a, 0, code_b, 0] | 0x6400 in each half = 1024 + code
                const uint32_t sel = (uint32_t)byte | 0x0C000000u | ((uint32_t)(4 + byte) << 16) | 0x00000C00u;
                const uint32_t x = __builtin_amdgcn_perm(xb, xa, sel) | 0x64006400u;
                bw[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h_t, x) + __builtin_bit_cast(v2h_t, zc[i]));
            }
            const v8h_t B = __builtin_bit_cast(v8h_t, v4u_t{bw[0], bw[1], bw[2], bw[3]});
#pragma unroll
            for (int S = 0; S < NSET; ++S)
                st.acc[S][sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[S], B, st.acc[S][sl], 0, 0, 0);
        }
    }
}

// Fold an int4 wave state into the workgroup's LDS layout (per wave and
// head: M, S, acc[128]).
template <int NSET>
__device__ __forceinline__ void mwave4_to_lds(MSmem4& sm, MState4<NSET>& st, int G, int lane, int wave) {
    const int g = lane >> 4;
    const int m = lane & 15;
    const float unscale = exp2i(-st.E);
#pragma unroll
    for (int S = 0; S < NSET; ++S) {
        float Ssum = st.S[S];
        Ssum += swz_xor16(Ssum);
        Ssum += xor32(Ssum);
        const int Hs = 4 * S + (m >> 2);
        if (g == 0 && (m & 3) == 0 && Hs < G) {
            sm.m[wave][Hs] = st.M[S];
            sm.s[wave][Hs] = Ssum;
        }
        const int H = 4 * S + g;
        if (H < G) {
            const int r0 = 2 * (m >> 3);
            float o[8];
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                const float hi = (m >> 3) ? st.acc[S][sl][2] : st.acc[S][sl][0];
                const float lo = (m >> 3) ? st.acc[S][sl][3] : st.acc[S][sl][1];
                o[sl] = (hi + lo) * unscale;
            }
            (void)r0;
            float4* dst = reinterpret_cast<float4*>(&sm.acc[wave][H][8 * m]);
            dst[0] = make_float4(o[0], o[1], o[2], o[3]);
            dst[1] = make_float4(o[4], o[5], o[6], o[7]);
        }
    }
}

// One workgroup = (sequence, kv-head, chunk) of either pool: chunks
// [0, r4.max_chunks) cover the int4 region, the rest the int8 window.
// Two head sets keep twice the accumulators: one wave per SIMD, no spills.
template <int NSET, bool BS8>
__global__ __launch_bounds__(kWGThreads, NSET == 2 ? 1 : 2) void kvq4_decode_mfma_kernel(DecodeArgs a) {
    __shared__ MSmem4 sm;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int m = lane & 15;
    const int G = a.nq / a.nkv;

    const int nct = n_chunks_total(a);
    const int wg = blockIdx.x;
    const int rest = wg >> 3;
    const int kh = rest % a.nkv;
    const int p = (rest / a.nkv) * 8 + (wg & 7);
    const int b = p / nct;
    const int c = p - b * nct;
    if (b >= a.batch) return;
    const bool int4_region = c < a.r4.max_chunks;
    const Region& reg = int4_region ? a.r4 : a.r8;
    const int cr = int4_region ? c : c - a.r4.max_chunks;
    const int chunk_len = a.tiles_per_wave * kChunkUnit;
    const int c0 = cr * chunk_len;
    const int32_t* btb = reg.bt + (size_t)b * reg.max_blocks;
    const int first = c0 + wave * kTile;
    const float4 qx = load_q4(a.q + ((size_t)b * a.nq + (size_t)kh * G) * kHD, G);
    int raw = mtile_raw(reg, btb, first, a.log2_bs, lane);
    const int L = effective_len(reg, b, a.log2_bs);
    if (c0 >= L) return;                                       // uniform per workgroup
    const int end = min(L, c0 + chunk_len);
    const int n_tiles = first < end ? (end - first + kChunkUnit - 1) / kChunkUnit : 1;

    if (int4_region) {
        const LaneOff4 lo = lane_offsets4(a, lane);
        MTile4 A, B;
        mtile4_issue<BS8>(a, raw, first, kh, lane, lo, A);
        raw = mtile_raw(reg, btb, first + kChunkUnit, a.log2_bs, lane);
        __asm__ volatile("" ::: "memory");
        quantize_q4(qx, G, sm.q);
        lds_barrier();
        const MQuery4 Q = load_q4_operand<NSET>(sm.q, G, g, m);
        MState4<NSET> st;
#pragma unroll
        for (int S = 0; S < NSET; ++S) {
            st.M[S] = -INFINITY;
            st.S[S] = 0.0f;
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) st.acc[S][sl] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        st.E = 100;
        int base = first;
        for (int k = 0;;) {
            if (k + 1 >= n_tiles) {
                mtile4_compute<NSET>(a, A, base, L, lane, wave, Q, st, sm);
                break;
            }
            mtile4_issue<BS8>(a, raw, base + kChunkUnit, kh, lane, lo, B);
            raw = mtile_raw(reg, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
            mtile4_compute<NSET>(a, A, base, L, lane, wave, Q, st, sm);
            base += kChunkUnit;
            ++k;
            if (k + 1 >= n_tiles) {
                mtile4_compute<NSET>(a, B, base, L, lane, wave, Q, st, sm);
                break;
            }
            mtile4_issue<BS8>(a, raw, base + kChunkUnit, kh, lane, lo, A);
            raw = mtile_raw(reg, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
            mtile4_compute<NSET>(a, B, base, L, lane, wave, Q, st, sm);
            base += kChunkUnit;
            ++k;
        }
        mwave4_to_lds<NSET>(sm, st, G, lane, wave);
        lds_barrier();
        mcombine_write(a, sm, G, b, kh, c);
    } else {
        const LaneOff lo = lane_offsets(a, lane);
        MTile A, B;
        mtile_issue<BS8>(a, raw, first, kh, lane, lo, A);
        raw = mtile_raw(reg, btb, first + kChunkUnit, a.log2_bs, lane);
        __asm__ volatile("" ::: "memory");
        quantize_q4(qx, G, sm.q);
        lds_barrier();
        const MQuery Q = load_q_operand(sm.q, G, g, m);
        MState st;
        st.M = -INFINITY;
        st.S = 0.0f;
        st.E = 100;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) st.acc[sl] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
        int base = first;
        for (int k = 0;;) {
            if (k + 1 >= n_tiles) {
                mtile_compute(a, A, base, L, lane, wave, Q, st, sm);
                break;
            }
            mtile_issue<BS8>(a, raw, base + kChunkUnit, kh, lane, lo, B);
            raw = mtile_raw(reg, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
            mtile_compute(a, A, base, L, lane, wave, Q, st, sm);
            base += kChunkUnit;
            ++k;
            if (k + 1 >= n_tiles) {
                mtile_compute(a, B, base, L, lane, wave, Q, st, sm);
                break;
            }
            mtile_issue<BS8>(a, raw, base + kChunkUnit, kh, lane, lo, A);
            raw = mtile_raw(reg, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
            mtile_compute(a, B, base, L, lane, wave, Q, st, sm);
            base += kChunkUnit;
            ++k;
        }
        mwrite_partial(a, sm, st, G, b, kh, c, lane, wave);
    }
}

template <bool BS8>
inline void launch_mfma4_bs(const DecodeArgs& a, int n_wg, hipStream_t s) {
    const dim3 grid(n_wg), block(kWGThreads);
    if (a.nq / a.nkv > 4)
        hipLaunchKernelGGL((kvq4_decode_mfma_kernel<2, BS8>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((kvq4_decode_mfma_kernel<1, BS8>), grid, block, 0, s, a);
}

inline void launch_mfma4(const DecodeArgs& a, int n_wg, hipStream_t s) {
    if (a.log2_bs < 4)
        launch_mfma4_bs<true>(a, n_wg, s);
    else
        launch_mfma4_bs<false>(a, n_wg, s);
}

// Enqueue the chunk kernel (if there is any context) and the merge kernel.
// new_dtype >= 0 fuses the write path of each sequence's last token.  The
// int8 cache and the mixed int4 / int8 cache both run on the matrix cores.
inline int launch_decode(const DecodeArgs& a, float* out, hipStream_t s, int new_dtype = -1) {
    const int nct = n_chunks_total(a);
    if (nct > 0) {
        const long pairs = (long)a.batch * nct;
        const long n_wg = (long)a.nkv * ((pairs + 7) / 8) * 8;
        if (n_wg > 0x7FFFFFFFL) return KVQ8_ESHAPE;
        if (a.r4.max_chunks > 0)
            launch_mfma4(a, (int)n_wg, s);
        else
            launch_mfma(a, (int)n_wg, new_dtype, s);
    }
    hipLaunchKernelGGL(kvq_merge_kernel<>, dim3(a.batch * a.nq), dim3(kMergeThreads), 0, s, out, a);
    return launch_status();
}


}  // namespace kvq
