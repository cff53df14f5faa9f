// int8 decode chunk kernel on the matrix cores ([P3] Sec. 2 seg. 1-3,
// generalized to batches, paged blocks and up to 8 query heads per kv-head).
//
// A wave processes tiles of 64 tokens of one kv-head.  Lane = (g, m) with
// g = lane / 16 and m = lane % 16; the 64 tokens of a tile form four groups
// of 16 (index v).
//
// Q.K: one v_mfma_i32_16x16x64_i8 per (token group v, row half h):
//   A = key codes   A[i][k] = K[token 16v+i][64h + k]   (lane holds 16 bytes)
//   B = query codes B[k][c] = Q[head c/2][64h + k] if 64h+k lies in 32-block
//                              2h + (c & 1), else 0
// so column c of the result is the int32 block dot product of block
// 2h + (c&1) for head c/2: one instruction gives two blocks of up to eight
// heads.  Lane (g, m) receives the dots of tokens 16v + 4g + r (r = 0..3) for
// column m; the per-block query scales are applied in float and the two
// block parities of a head meet with one DPP step (lanes m, m^1).
//
// Softmax: lane (g, m) owns the 16 scores of head m/2 for tokens
// 16v + 4g + r; the tile max is a 16-value max and two cross-row steps.
//
// P.V: one v_mfma_f32_16x16x32_f16 per (pair of token groups, d-slice s):
//   A = weights  A[c][k]: row c = head c/2, the f16 high part of
//                p * vstep for even c and the remainder below it (rounded
//                toward zero) for odd c (together within 2^-21 relative)
//   B = values   B[k][m] = V[token k][8m + s] as f16 (exact for int8)
// The weights are exactly the lane's own scores' tokens, so no data moves
// between the two products.  Lane (g, m) accumulates rows 4g..4g+3 = heads
// 2g, 2g+1 (high and low part each) at d = 8m + s.
#pragma once

#include "kvq_decode_core.h"

namespace kvq {

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));

constexpr int kMGroup = 8;         // query heads per kv-head handled by the MFMA kernel

// One tile in operand layout (native vector types: selects on them stay in
// registers).
struct MTile {
    v4u_t k[4][2];     // [v][h]: token 16v+m, bytes 64h+16g .. +15
    v2u_t v[4][4];     // [v][e]: token 16v+4g+e, bytes 8m .. 8m+7
    float ks, vs;      // steps of token base+lane
    int id;            // block id of token base+lane, -1 if outside the pool
};

struct MQuery {
    v4i_t op[2];       // B operand of the Q.K product, per row half
    float sc[2];       // query block scale of column m, per row half
};

struct MState {
    float M;           // running max of head m/2 (base-2 units)
    float S;           // this lane's share of the running sum of head m/2
    int E;             // the accumulator holds its value times 2^E (wave-uniform)
    v4f_t acc[8];      // [slice s]: rows 4g+r at d = 8m+s
};

// LDS of one workgroup.
struct MSmem {
    QSmem q;                           // query codes and block scales
    float ks[kWaves][64];              // key step * score scale (0 if masked)
    float kb[kWaves][64];              // 0, or -inf for a masked token
    float vs[kWaves][64];              // value step (0 if masked)
    v4u_t nk[8], nv[8];                // fused write path: the new token's codes
    float nstep[2];
    float acc[kWaves][kMGroup][kHD];   // per-wave accumulators for the merge
    float m[kWaves][kMGroup];
    float s[kWaves][kMGroup];
};

typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));

// two floats to f16, round toward zero (used where the values are exact)
__device__ __forceinline__ uint32_t pack_f16_rtz(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// The value weights enter the f16 products in two parts: rows with even
// index take the high part of each weight (its f16 rounding toward zero: the
// top 11 significant bits), rows with odd index the f16 of the remainder
// below it (rounded toward zero: within 2^-10 of the remainder, so the two
// together are within 2^-21 of the weight).  part_mask is all-zero for the
// even rows and keeps the top 11 significant bits for the odd ones, so one
// masked subtraction per weight gives either part and the conversion is the
// same instruction for both.
__device__ __forceinline__ uint32_t weight_part_mask(int m) { return (m & 1) ? 0xFFFFE000u : 0u; }

__device__ __forceinline__ uint32_t weight_part_f16x2(float w0, float w1, uint32_t part_mask) {
    return pack_f16_rtz(w0 - __uint_as_float(__float_as_uint(w0) & part_mask),
                        w1 - __uint_as_float(__float_as_uint(w1) & part_mask));
}

__device__ __forceinline__ float bperm_f(float v, int src_lane) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}

__device__ __forceinline__ MQuery load_q_operand(const QSmem& sm, int G, int g, int m) {
    MQuery Q;
    const int H = m >> 1;
    const bool live = H < G;
    const bool mine = live && ((g >> 1) == (m & 1));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const v4u_t c = *reinterpret_cast<const v4u_t*>(&sm.qc[H][16 * h + 4 * g]);
        Q.op[h] = mine ? __builtin_bit_cast(v4i_t, c) : v4i_t{0, 0, 0, 0};
        const float s = sm.qs[H][2 * h + (m & 1)];
        Q.sc[h] = live ? s : 0.0f;
    }
    return Q;
}

// Value codes are read with the non-temporal (streaming) cache policy, keys
// with the default one.  Each value line is used by exactly one wave, once;
// measured on MI355X (interleaved runs on one box), streaming the values took
// the batch-32 layer from 193.7 to 178.5 us and the 8K batch-1 step from 303.5
// to 284.0 us, while streaming the keys as well made both slower (keys only:
// slower still).
__device__ __forceinline__ v2u_t load_value_nt(const int8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v2u_t*>(p));
}

// Table entry of the tile's token base+lane (clamped index: always in bounds).
__device__ __forceinline__ int mtile_raw(const Region& r, const int32_t* __restrict__ btb, int base, int log2_bs,
                                         int lane) {
    return btb[min((base + lane) >> log2_bs, r.max_blocks - 1)];
}

// Lane parts of the load addresses (bytes from the start of the token
// group's first slot row), fixed for the whole kernel: the key row of token
// 16v+m, bytes 16g.., and the value rows of tokens 16v+4g+e, bytes 8m.., each
// at the column where kv-head kh is stored in that token's slot (the pool's
// storage order, q8_col: a token's slot index modulo 8 is its lane's token
// index modulo 8, since token groups start on block boundaries).
struct LaneOff {
    uint32_t k;
    uint32_t v[4];
    uint32_t kc;       // the key column alone (bytes), for 8-slot blocks
    uint32_t vc[4];
};

__device__ __forceinline__ LaneOff lane_offsets(const DecodeArgs& a, int lane, int kh) {
    const int g = lane >> 4;
    const int m = lane & 15;
    const uint32_t row = (uint32_t)a.nkv * kHD;        // bytes between consecutive slots
    const int p = q8_rot_group(a.nkv);
    LaneOff o;
    o.kc = (uint32_t)q8_col(kh, m, p) * kHD;
    o.k = (uint32_t)m * row + 16 * g + o.kc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o.vc[e] = (uint32_t)q8_col(kh, 4 * g + e, p) * kHD;
        o.v[e] = (uint32_t)(4 * g + e) * row + 8 * m + o.vc[e];
    }
    return o;
}

// Which loads of a tile to issue: keys, values, steps.  A tile walk issues
// keys and steps of the next tile before the current tile's Q.K and its
// values after it, when the current keys are dead, so that two full tiles
// are never held in registers at once.
enum : int { kIssueKeys = 1, kIssueValues = 2, kIssueSteps = 4, kIssueAll = 7 };

// Issue loads of a tile.  Rows of invalid blocks read slot 0 of the pool
// (in bounds) and are masked when the tile is computed.  Row indices (in head
// rows of 128 B) fit in 32 bits: the host rejects larger pools.  A call
// without kIssueKeys takes the block ids from T.id, set by an earlier call
// for the same tile.
//
// With blocks of 16 or more slots a 16-token group lies in one block, so its
// base address is wave-uniform and the lane parts are fixed (scalar base +
// 32-bit lane offset).  With 8-slot blocks each lane picks one of the two
// blocks of its group.
template <bool BS8, int PARTS = kIssueAll>
__device__ __forceinline__ void mtile_issue(const DecodeArgs& a, int raw, int base, int kh, int lane,
                                            const LaneOff& lo, MTile& T) {
    constexpr bool KEYS = PARTS & kIssueKeys, VALUES = PARTS & kIssueValues, STEPS = PARTS & kIssueSteps;
    const int g = lane >> 4;
    const int m = lane & 15;
    const uint32_t bs_mask = (1u << a.log2_bs) - 1;
    int id;
    if constexpr (KEYS) {
        id = (raw >= 0 && raw < a.r8.n_blocks) ? raw : -1;
        T.id = id;
    } else {
        id = T.id;
    }
    const uint32_t nkv = (uint32_t)a.nkv;
    // slot row (slot * nkv) of the first token of 8-token group i
    // (wave-uniform; the lane offsets add the head's column); each value is
    // computed where it is used so that a per-lane choice between two groups
    // stays a select and never becomes an indexed array
    auto grp = [&](int i) __attribute__((always_inline)) -> uint32_t {
        const int idi = __builtin_amdgcn_readlane(id, 8 * i);
        // a block outside the pool reads block 0 (in bounds; its tokens are masked)
        const uint32_t idc = (uint32_t)max(idi, 0);
        return ((idc << a.log2_bs) + (((uint32_t)base + 8 * i) & bs_mask)) * nkv;
    };
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        if constexpr (!BS8) {
            const uint32_t u = grp(2 * v);
            if constexpr (KEYS) {
                const int8_t* pk = a.kc + (size_t)u * kHD;
                T.k[v][0] = *reinterpret_cast<const v4u_t*>(pk + lo.k);
                T.k[v][1] = *reinterpret_cast<const v4u_t*>(pk + lo.k + 64);
            }
            if constexpr (VALUES) {
                const int8_t* pv = a.vc + (size_t)u * kHD;
#pragma unroll
                for (int e = 0; e < 4; ++e) T.v[v][e] = load_value_nt(pv + lo.v[e]);
            }
        } else {
            const uint32_t u0 = grp(2 * v), u1 = grp(2 * v + 1);
            if constexpr (KEYS) {
                const uint32_t rk = ((m & 8) ? u1 : u0) + (uint32_t)(m & 7) * nkv;
                const int8_t* p = a.kc + (size_t)rk * kHD + 16 * g + lo.kc;
                T.k[v][0] = *reinterpret_cast<const v4u_t*>(p);
                T.k[v][1] = *reinterpret_cast<const v4u_t*>(p + 64);
            }
            if constexpr (VALUES) {
                const uint32_t rv = ((g & 2) ? u1 : u0) + (uint32_t)(4 * (g & 1)) * nkv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    T.v[v][e] = load_value_nt(a.vc + (size_t)(rv + (uint32_t)e * nkv) * kHD + 8 * m + lo.vc[e]);
            }
        }
    }
    if constexpr (STEPS) {
        const uint32_t srow =
            id >= 0 ? ((((uint32_t)id << a.log2_bs) + (((uint32_t)base + lane) & bs_mask)) * nkv + kh) : 0u;
        T.ks = a.ks[srow];
        T.vs = a.vs[srow];
    }
}

// Fused write path: the new token's codes (LDS) replace the tile's stale copy
// of its slot, so the tile is computed exactly as after a separate write.
// Every select tests the lane's own token index against tn.
__device__ __forceinline__ MTile mtile_substitute(MTile T, const MSmem& sm, int base, int tn, int lane) {
    const int g = lane >> 4;
    const int m = lane & 15;
    const v4u_t k0 = sm.nk[g], k1 = sm.nk[4 + g];
    const v4u_t c = sm.nv[m >> 1];
    const v2u_t cv = (m & 1) ? v2u_t{c.z, c.w} : v2u_t{c.x, c.y};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const bool kme = base + 16 * v + m == tn;
        T.k[v][0] = kme ? k0 : T.k[v][0];
        T.k[v][1] = kme ? k1 : T.k[v][1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool vme = base + 16 * v + 4 * g + e == tn;
            T.v[v][e] = vme ? cv : T.v[v][e];
        }
    }
    const bool sme = base + lane == tn;
    T.ks = sme ? sm.nstep[0] : T.ks;
    T.vs = sme ? sm.nstep[1] : T.vs;
    return T;
}

// The int32 block dot products of a tile: d[v][h][r] is, for lane (g, m),
// the dot of block 2h + (m & 1) of head m/2 with token 16v + 4g + r.
__device__ __forceinline__ void mtile_qk(const MTile& T, const MQuery& Q, v4i_t (&d)[4][2]) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            d[v][h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i_t, T.k[v][h]), Q.op[h],
                                                            v4i_t{0, 0, 0, 0}, 0, 0, 0);
}

// Maximum over the whole wave, in every lane.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    return group8_max(v);
}

// 2^e as a float for e <= 127; 0 below the normal range (a rescale factor
// that small only ever meets an accumulator of zeros or negligible terms)
__device__ __forceinline__ float exp2i(int e) {
    return e < -126 ? 0.0f : __uint_as_float((uint32_t)(e + 127) << 23);
}

// Byte `byte` of two words of int8 codes as an f16 pair (low half from wa),
// exactly: the byte with its sign bit flipped is code + 128, which as the
// mantissa of 2^10 gives the f16 1152 + code; one packed f16 subtraction of
// 1152 leaves the code.
__device__ __forceinline__ uint32_t codes_f16x2(uint32_t wa, uint32_t wb, int byte) {
    const uint32_t sel = (uint32_t)byte | 0x00000C00u | ((uint32_t)(4 + byte) << 16) | 0x0C000000u;
    const uint32_t x = __builtin_amdgcn_perm(wb, wa, sel) ^ 0x64806480u;
    const v2h_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h_t, x) + bias);
}

// One tile.
//
// The value weights p * vstep enter the f16 product as a high part (11
// significant bits, exact in f16) and the remainder below it rounded toward
// zero: within 2^-21 relative.  To keep them in f16 range they carry a wave-wide power of
// two 2^E with max(vstep) * 2^E < 2^15; E only ever decreases, and the
// accumulator holds its value times 2^E.
struct NoHook {
    __device__ void operator()() const {}
};

// `after_qk` runs once the tile's keys are consumed (the walk issues the next
// tile's value loads there).
template <class Hook = NoHook, class Hook2 = NoHook>
__device__ __forceinline__ void mtile_compute(const DecodeArgs& a, const MTile T, int base, int L, int lane,
                                              int wave, const MQuery& Q, MState& st, MSmem& sm,
                                              Hook after_qk = Hook(), Hook2 after_pv = Hook2()) {
    const int g = lane >> 4;
    const int m = lane & 15;
    // steps through LDS: lane l holds token base+l, the products need tokens
    // 16v + 4g + r
    {
        const bool ok = (base + lane < L) && T.id >= 0;
        const float vsv = ok ? T.vs : 0.0f;
        const float vm = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(vsv))));
        if (vm > 0.0f) {
            const int e = (int)((__float_as_uint(vm) >> 23) & 0xFFu) - 127;
            const int Et = min(max(14 - e, -100), 100);
            if (Et < st.E) {
                const float f = exp2i(Et - st.E);
#pragma unroll
                for (int sl = 0; sl < 8; ++sl) st.acc[sl] *= f;
                st.E = Et;
            }
        }
        sm.ks[wave][lane] = ok ? T.ks * a.score_scale : 0.0f;
        sm.kb[wave][lane] = ok ? 0.0f : -INFINITY;
        sm.vs[wave][lane] = vsv * exp2i(st.E);
    }
    float s[4][4];
    {
        v4i_t d[4][2];
        mtile_qk(T, Q, d);
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float f = (float)d[v][0][r] * Q.sc[0];
                f = fmaf((float)d[v][1][r], Q.sc[1], f);
                s[v][r] = f + dpp_f<kDppXor1>(f);
            }
    }
    after_qk();
    float mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float4 kk = *reinterpret_cast<const float4*>(&sm.ks[wave][16 * v + 4 * g]);
        const float4 kb = *reinterpret_cast<const float4*>(&sm.kb[wave][16 * v + 4 * g]);
        const float k4[4] = {kk.x, kk.y, kk.z, kk.w};
        const float b4[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[v][r] = fmaf(s[v][r], k4[r], b4[r]);
            mt = fmaxf(mt, s[v][r]);
        }
    }
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
    }
    // a head whose tokens so far are all masked keeps M = -inf: its weights
    // must come out 0, not exp2(-inf - -inf)
    const float mref = (st.M == -INFINITY) ? 0.0f : st.M;
    const uint32_t part_mask = weight_part_mask(m);
    uint32_t wop[4][2];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float4 vv = *reinterpret_cast<const float4*>(&sm.vs[wave][16 * v + 4 * g]);
        const float v4[4] = {vv.x, vv.y, vv.z, vv.w};
        float w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(s[v][r] - mref);
            st.S += p;
            w[r] = p * v4[r];
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            wop[v][pr] = weight_part_f16x2(w[2 * pr], w[2 * pr + 1], part_mask);
        }
    }
#pragma unroll
    for (int vp = 0; vp < 2; ++vp) {
        const v8h_t A = __builtin_bit_cast(
            v8h_t, v4u_t{wop[2 * vp][0], wop[2 * vp][1], wop[2 * vp + 1][0], wop[2 * vp + 1][1]});
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            uint32_t bw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q0 = 2 * i, q1 = 2 * i + 1;      // element q: token group 2vp + q/4, e = q%4
                const v2u_t c0 = T.v[2 * vp + q0 / 4][q0 % 4];
                const v2u_t c1 = T.v[2 * vp + q1 / 4][q1 % 4];
                bw[i] = codes_f16x2(sl < 4 ? c0.x : c0.y, sl < 4 ? c1.x : c1.y, sl & 3);
            }
            const v8h_t B = __builtin_bit_cast(v8h_t, v4u_t{bw[0], bw[1], bw[2], bw[3]});
            st.acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, st.acc[sl], 0, 0, 0);
        }
    }
    after_pv();
}

// Fold the waves' states (in LDS: per wave M, S and acc of each head) and
// write one partial per query head.
template <class Args>
__device__ __forceinline__ void mcombine_write(const Args& a, const MSmem& sm, int G, int b, int kh, int c) {
    const int nct = n_chunks_total(a);
    for (int idx = threadIdx.x; idx < G * kHD; idx += kWGThreads) {
        const int h = idx / kHD;
        const int d = idx - h * kHD;
        float M = sm.m[0][h];
#pragma unroll
        for (int wv = 1; wv < kWaves; ++wv) M = fmaxf(M, sm.m[wv][h]);
        float tot = 0.0f, ssum = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) {
                const float f = __builtin_amdgcn_exp2f(sm.m[wv][h] - M);
                tot = fmaf(sm.acc[wv][h][d], f, tot);
                ssum = fmaf(sm.s[wv][h], f, ssum);
            }
        }
        const size_t pi = ((size_t)b * a.nq + (size_t)kh * G + h) * nct + c;
        a.ws_acc[pi * kHD + d] = tot;
        if (d == 0) {
            a.ws_m[pi] = M;
            a.ws_s[pi] = ssum;
        }
    }
}

// Fold the wave states of the workgroup and write one partial per query head.
template <class Args>
__device__ __forceinline__ void mwrite_partial(const Args& a, MSmem& sm, MState& st, int G, int b, int kh,
                                               int c, int lane, int wave) {
    const int g = lane >> 4;
    const int m = lane & 15;
    float S = st.S;
    S += swz_xor16(S);
    S += xor32(S);
    if (g == 0 && (m & 1) == 0 && (m >> 1) < G) {
        sm.m[wave][m >> 1] = st.M;
        sm.s[wave][m >> 1] = S;
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int H = 2 * g + hh;
        if (H < G) {
            float o[8];
            const float unscale = exp2i(-st.E);
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) o[sl] = (st.acc[sl][2 * hh] + st.acc[sl][2 * hh + 1]) * unscale;
            float4* dst = reinterpret_cast<float4*>(&sm.acc[wave][H][8 * m]);
            dst[0] = make_float4(o[0], o[1], o[2], o[3]);
            dst[1] = make_float4(o[4], o[5], o[6], o[7]);
        }
    }
    lds_barrier();
    mcombine_write(a, sm, G, b, kh, c);
}

}  // namespace kvq
