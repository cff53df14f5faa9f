// Q4_0 KV mode ([P2] Sec. 1 and Sec. 3: the --kv-q4 switch, a Q4_0 payload
// cache about 1.65x denser than q8 whose decode dot product reads the nibbles
// without dequantizing them).
//
// Format, per (token, kv-head) row of 128 values: four blocks of 32, each
// with a float32 step = (the block's value of largest magnitude, the negative
// one on a sign tie) / -8, and 4-bit codes c = min(15, floor(x / step + 8.5))
// standing for (c - 8) * step; a block of zeros has step +0 and codes 8.
// 64 code bytes + 16 step bytes = 80 B per row against q8's 132 B.
//
// Byte layouts (chosen for the decode kernel's lanes):
//   key row:   byte j = code[j] | code[64 + j] << 4
//   value row: byte 4m + k = code[32k + 2m] | code[32k + 2m + 1] << 4
//
// Decode: the int8 path's matrix-core walk (see kvq_decode_mfma.h) with
//   Q.K  the nibbles of a key half-row as the i8 operand; the accumulator
//        input -8 * R (R = sum of the query block's codes) makes each column
//        the block term P - 8R; block term x query block scale x key block
//        step, the two parities of a head summed by one DPP step;
//   P.V  one v_mfma_f32_16x16x32_f16 per (pair of token groups, slice s):
//        columns m of slice s are d = 32(s/2) + 2m + (s & 1), all in value
//        block s/2, so the A operand holds the weights p * vstep of that
//        block (f16 high part + f16 remainder, rows = (head, part)) and B
//        holds c as f16 (exact; one fp8 -> f16 conversion per token pair);
//        a second product with B = -8 everywhere adds the -8 sum_t w_t of
//        the block.  Up to 8 heads in one operand set.
#include "kvq8.h"
#include "kvq_decode_mfma.h"

namespace kvq {

// ----------------------------------------------------------------------------
// write path
// ----------------------------------------------------------------------------

// Rows per 8-lane group; a 256-thread workgroup quantizes 128 rows.
constexpr int kQ40RowsPerGroup = 4;
constexpr int kQ40RowsPerBlock = 32 * kQ40RowsPerGroup;

// A row of 128 values is spread over 8 lanes, 16 values each: block k's
// first half (values 32k .. 32k + 15) on lane k, its second half on lane
// 7 - k.  A block's extreme is then one half-row mirror, key bytes pair
// lanes 2 apart (blocks k and k + 2, same half) and each quad holds one half
// of all four blocks (lanes 0..3 in block order, lanes 4..7 reversed).
//
// Codes of a lane's 16 values, one byte each (c[h] holds values 4h .. 4h + 3),
// and its block's step.
//
// The block extreme is the value of largest magnitude, the negative one on a
// tie: the largest of the keys rotl(bits, 1) (magnitude above, sign in bit
// 0) as unsigned integers.
//
// The code is floor(x / step + 8.5) clamped to 15.  f = fma(x, rcp(step),
// 136.5 + 2^-15) lies in [128, 256), so its unit is 2^-16: the mantissa is
// (x * rcp(step) + 8.5) * 2^16, rounded, plus 2.  Bits 16..23 of f are then
// the code (the exponent's low bit is 0) and bits 0..15 the fraction plus 2.
// Where those low bits are 0..3 the quotient + 8.5 lies within 2^-15 of an
// integer and the lane divides instead (about 0.01% of the values, and every
// value of a zero block, whose quotients are NaN).  Elsewhere it lies at
// least 1.5 * 2^-16 from one, far more than one rcp error (8 * 2^-23) plus
// the division's and the addition's roundings, so the floor read from f is
// the floor of the correctly rounded x / step + 8.5.  A zero block has step
// +0 and codes 8.  Four code bytes are gathered by two byte permutes, and
// the one code that can reach 16 (q >= 7.5) is brought to 15 on the packed
// word.
__device__ __forceinline__ void q40_quantize16(const float (&x)[16], uint32_t (&c)[4], float& step) {
#pragma clang fp contract(off)
    constexpr float kMagic = 136.500030517578125f;   // 128 + 8.5 + 2^-15
    uint32_t km = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const uint32_t u = __float_as_uint(x[e]);
        km = max(km, __builtin_amdgcn_alignbit(u, u, 31u));   // rotl(u, 1)
    }
    km = max(km, (uint32_t)dpp_i<kDppHalfMirror>((int)km));   // the block's other lane
    const float m = __uint_as_float(__builtin_amdgcn_alignbit(km, km, 1u));   // rotr(km, 1)
    step = km < 2u ? 0.0f : m * -0.125f;             // exact: a power-of-two division
    const float rs = __builtin_amdgcn_rcpf(step);
    uint32_t cb[16];                                 // byte 2: the code (16 for q >= 7.5)
    uint64_t slow[16];                               // wave masks of the lanes that divide
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        cb[e] = __float_as_uint(__builtin_fmaf(x[e], rs, kMagic));
        slow[e] = __builtin_amdgcn_ballot_w64((uint16_t)cb[e] <= 3u);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (slow[e] != 0) {                         // rare: one wave-uniform test per value
            const float cd = step == 0.0f ? 8.0f : fminf(floorf(x[e] / step + 8.5f), 15.0f);
            cb[e] = ((slow[e] >> (threadIdx.x & 63)) & 1) ? (uint32_t)(int)cd << 16 : cb[e];
        }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const uint32_t v = __builtin_amdgcn_perm(cb[4 * h + 1], cb[4 * h], 0x0C0C0602u) |
                           __builtin_amdgcn_perm(cb[4 * h + 3], cb[4 * h + 2], 0x06020C0Cu);
        c[h] = v - ((v >> 4) & 0x01010101u);         // 16 -> 15, codes 0..15 unchanged
    }
}

// Byte selectors of the quad gather of value bytes, fixed per lane: the lane
// at quad position q builds the value word whose byte k comes from byte q of
// the word W held by the quad lane of block k (position k, or 3 - k in the
// second quad of the 8-lane group).  Sources are W itself and W of the lanes
// q + 1, q + 2, q + 3 (mod 4), two per byte permute.
struct Q40Gather {
    uint32_t lo, hi;     // selectors over (W of lane q + 1 : W) and (W of lane q + 3 : W of lane q + 2)
};

__device__ __forceinline__ Q40Gather q40_gather_selectors(int q, bool reversed) {
    Q40Gather s{0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int src = reversed ? 3 - k : k;
        const int j = (src - q) & 3;
        const uint32_t b = (uint32_t)((j & 1) ? 4 + q : q);
        s.lo |= (j < 2 ? b : 0x0Cu) << (8 * k);
        s.hi |= (j >= 2 ? b : 0x0Cu) << (8 * k);
    }
    return s;
}

__device__ __forceinline__ uint32_t q40_value_word(uint32_t W, const Q40Gather& s) {
    const uint32_t q1 = (uint32_t)dpp_i<kDppQuadRot1>((int)W);   // lane q + 1
    const uint32_t q2 = (uint32_t)dpp_i<kDppXor2>((int)W);       // lane q + 2
    const uint32_t q3 = (uint32_t)dpp_i<kDppQuadRot3>((int)W);   // lane q + 3
    return __builtin_amdgcn_perm(q1, W, s.lo) | __builtin_amdgcn_perm(q3, q2, s.hi);
}

// One (token, kv-head, K-or-V) row per 8 lanes, 4 rows per 8-lane group;
// a wave quantizes only key rows or only value rows (kind = wave & 1).
// Pool rows (head-major, hm_row) fit in 32 bits: the host checks n_slots *
// nkv, and ns_cap = min(n_slots, 2^31) turns the slot test into one
// unsigned compare.
template <int DT>
__global__ __launch_bounds__(256) void kvq4_0_quantize_append_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs,
    uint32_t ns_cap, DivN nkv, int log2_bs, const void* __restrict__ k_new,
    const void* __restrict__ v_new, int n_rows, const int32_t* __restrict__ slots) {
    constexpr int kInBytes = DT == KVQ8_F32 ? 4 : 2;
    const int l8 = threadIdx.x & 7;
    const int half = l8 >> 2;                      // 0: first halves of the blocks, 1: second halves
    const int q = l8 & 3;                          // quad position
    const int kb = half ? 3 - q : q;               // block of the lane's values
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int kind = wave & 1;                     // 0: key rows, 1: value rows
    const int g8 = (threadIdx.x >> 3) & 7;         // 8-lane group in the wave
    const void* src = kind ? v_new : k_new;
    uint8_t* codes = kind ? vc : kc;
    float* steps = kind ? vs : ks;
    const uint32_t in_off = (uint32_t)(32 * kb + 16 * half) * kInBytes;
    const Q40Gather gsel = q40_gather_selectors(q, half != 0);
    Raw16<DT> raw[kQ40RowsPerGroup];
    int khs[kQ40RowsPerGroup];
    uint32_t slot[kQ40RowsPerGroup];
    // rows past the end load the last row again and store nothing; indices
    // fit in 32 bits (the host checks the row count).  Pairs are token-major
    // (pair = token * nkv + kv-head), so a wave reads one contiguous run of
    // input rows (the kv-head-major order of the int4 writers measured 9%
    // slower here).
#pragma unroll
    for (int k = 0; k < kQ40RowsPerGroup; ++k) {
        const int pair = (int)blockIdx.x * (kQ40RowsPerBlock / 2) + ((wave >> 1) * 8 + g8) * kQ40RowsPerGroup + k;
        const int tr = min(2 * pair + kind, n_rows - 1) >> 1;   // token * nkv + kv-head
        const int tok = div_n(tr, nkv);
        khs[k] = tr - tok * nkv.n;
        load_raw16<DT>(src, (size_t)tr * (kHD * kInBytes) + in_off, raw[k]);
        slot[k] = (uint32_t)slots[tok];
    }
#pragma unroll
    for (int k = 0; k < kQ40RowsPerGroup; ++k) {
        const int pair = (int)blockIdx.x * (kQ40RowsPerBlock / 2) + ((wave >> 1) * 8 + g8) * kQ40RowsPerGroup + k;
        float x[16];
        unpack_raw16<DT>(raw[k], x);
        uint32_t c[4];
        float step;
        q40_quantize16(x, c, step);                 // both lanes of a block take part (DPP)
        uint32_t w0, w1;
        uint32_t off;
        if (kind == 0) {
            // key byte j = code[j] | code[64 + j] << 4: blocks k and k + 2 of
            // one half are quad lanes q and q ^ 2; the block 0 / 1 lane
            // writes the low 8 of their 16 bytes, its partner the high 8
            const bool low = kb < 2;
            const uint32_t r0 = (uint32_t)dpp_i<kDppXor2>((int)(low ? c[2] : c[0]));
            const uint32_t r1 = (uint32_t)dpp_i<kDppXor2>((int)(low ? c[3] : c[1]));
            w0 = low ? (c[0] | (r0 << 4)) : (r0 | (c[2] << 4));
            w1 = low ? (c[1] | (r1 << 4)) : (r1 | (c[3] << 4));
            off = 32u * (uint32_t)(kb & 1) + 16u * (uint32_t)half + (low ? 0u : 8u);
        } else {
            // value byte 4m + kb = code[32 kb + 2m] | code[32 kb + 2m + 1] << 4:
            // the lane's pairs m = 8 half .. 8 half + 7 of block kb, then one
            // byte of every block per word: words m = 8 half + q and m + 4
            uint32_t a[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) a[h] = c[h] | (c[h] >> 4);   // bytes 0, 2: the pairs
            w0 = q40_value_word(__builtin_amdgcn_perm(a[1], a[0], 0x06040200u), gsel);
            w1 = q40_value_word(__builtin_amdgcn_perm(a[3], a[2], 0x06040200u), gsel);
            off = 32u * (uint32_t)half + 4u * (uint32_t)q;
        }
        if (2 * pair + kind >= n_rows || slot[k] >= ns_cap) continue;   // uniform per 8-lane row
        const uint32_t drow = hm_row32(slot[k], (uint32_t)khs[k], (uint32_t)nkv.n, log2_bs);
        uint8_t* dst = codes + (size_t)drow * (kHD / 2) + off;
        if (kind == 0) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
        } else {
            *reinterpret_cast<uint32_t*>(dst) = w0;
            *reinterpret_cast<uint32_t*>(dst + 16) = w1;
        }
        if (half == 0) steps[(size_t)drow * 4 + kb] = step;
    }
}

// ----------------------------------------------------------------------------
// decode
// ----------------------------------------------------------------------------

constexpr int kQ40RowBytes = kHD / 2;

// One tile in operand layout.
struct QTile {
    v4u_t k[4];          // [v]: token 16v+m, key bytes 16g .. 16g+15
    uint32_t v[4][4];    // [v][e]: token 16v+4g+e, value bytes 4m .. 4m+3
    v4f_t ks, vs;        // block steps of token base+lane
    int id;              // block id of token base+lane, -1 if outside the pool
};

struct QSmem40 : MSmem {
    float kst[kWaves][4][64];     // key block step * score scale (0 if masked)
    float vst[kWaves][4][64];     // value block step * 2^E (0 if masked)
};

// Lane parts of the load addresses (bytes) from the first row of a 16-token
// group, fixed for the whole kernel: a (block, kv-head)'s rows are
// contiguous in the head-major pool.
struct QLaneOff {
    uint32_t k;          // key row of token 16v+m, bytes 16g..
    uint32_t v[4];       // value rows of tokens 16v+4g+e, bytes 4m..
};

__device__ __forceinline__ QLaneOff q40_lane_offsets(int lane) {
    const int g = lane >> 4;
    const int m = lane & 15;
    QLaneOff o;
    o.k = (uint32_t)m * kQ40RowBytes + 16 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) o.v[e] = (uint32_t)(4 * g + e) * kQ40RowBytes + 4 * m;
    return o;
}

// Loads of a tile (the parts as for the int8 tile).  Codes live in a.k4 /
// a.v4 ([n_blocks][nkv][kv_bs][64]), steps in a.ks / a.vs
// ([n_blocks][nkv][kv_bs][4]), head-major (hm_row); rows of invalid blocks
// read block 0.
template <bool BS8, int PARTS = kIssueAll>
__device__ __forceinline__ void qtile_issue(const DecodeArgs& a, int raw, int base, int kh, int lane,
                                            const QLaneOff& lo, QTile& T) {
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
    auto grp = [&](int i) __attribute__((always_inline)) -> uint32_t {
        const int idi = __builtin_amdgcn_readlane(id, 8 * i);
        // a block outside the pool reads block 0 (in bounds; its tokens are masked)
        const uint32_t idc = (uint32_t)max(idi, 0);
        return ((idc * nkv + (uint32_t)kh) << a.log2_bs) + (((uint32_t)base + 8 * i) & bs_mask);
    };
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        if constexpr (!BS8) {
            const uint32_t u = grp(2 * v);
            if constexpr (KEYS)
                T.k[v] = *reinterpret_cast<const v4u_t*>(a.k4 + (size_t)u * kQ40RowBytes + lo.k);
            if constexpr (VALUES) {
                const uint8_t* pv = a.v4 + (size_t)u * kQ40RowBytes;
#pragma unroll
                for (int e = 0; e < 4; ++e) T.v[v][e] = *reinterpret_cast<const uint32_t*>(pv + lo.v[e]);
            }
        } else {
            const uint32_t u0 = grp(2 * v), u1 = grp(2 * v + 1);
            if constexpr (KEYS) {
                const uint32_t rk = ((m & 8) ? u1 : u0) + (uint32_t)(m & 7);
                T.k[v] = *reinterpret_cast<const v4u_t*>(a.k4 + (size_t)rk * kQ40RowBytes + 16 * g);
            }
            if constexpr (VALUES) {
                const uint32_t rv = ((g & 2) ? u1 : u0) + (uint32_t)(4 * (g & 1));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    T.v[v][e] = *reinterpret_cast<const uint32_t*>(
                        a.v4 + (size_t)(rv + (uint32_t)e) * kQ40RowBytes + 4 * m);
            }
        }
    }
    if constexpr (STEPS) {
        const uint32_t srow =
            id >= 0 ? ((((uint32_t)id * nkv + (uint32_t)kh) << a.log2_bs) + (((uint32_t)base + lane) & bs_mask)) : 0u;
        T.ks = *reinterpret_cast<const v4f_t*>(a.ks + (size_t)srow * 4);
        T.vs = *reinterpret_cast<const v4f_t*>(a.vs + (size_t)srow * 4);
    }
}

// -8 * (sum of the query codes of block 2h + (m & 1) of head m/2), per row
// half h: the accumulator input that turns the i8 product into P - 8R.
__device__ __forceinline__ void q40_block_bias(const QSmem& sm, int G, int m, int (&nr)[2]) {
    const int H = m >> 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int r = 0;
        if (H < G) {
            const int b = 2 * h + (m & 1);
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const uint32_t word = sm.qc[H][8 * b + w];
#pragma unroll
                for (int k = 0; k < 4; ++k) r += (int)(int8_t)(word >> (8 * k));
            }
        }
        nr[h] = -8 * r;
    }
}

// One tile (readings of the weights, E and masking as in mtile_compute).
template <class Hook = NoHook>
__device__ __forceinline__ void qtile_compute(const DecodeArgs& a, const QTile T, int base, int L, int lane,
                                              int wave, const MQuery& Q, const int (&nr)[2], MState& st,
                                              QSmem40& sm, Hook after_qk = Hook()) {
    const int g = lane >> 4;
    const int m = lane & 15;
    // steps through LDS: lane l holds token base+l, the products need tokens
    // 16v + 4g + r
    {
        const bool ok = (base + lane < L) && T.id >= 0;
        const v4f_t kv = ok ? T.ks : v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
        const v4f_t vv = ok ? T.vs : v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
        const float va = fmaxf(fmaxf(fabsf(vv.x), fabsf(vv.y)), fmaxf(fabsf(vv.z), fabsf(vv.w)));
        const float vm = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(va))));
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
        const float sc = exp2i(st.E);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            sm.kst[wave][b][lane] = kv[b] * a.score_scale;
            sm.vst[wave][b][lane] = vv[b] * sc;
        }
        sm.kb[wave][lane] = ok ? 0.0f : -INFINITY;
    }
    float s[4][4];
    {
        v4i_t d[4][2];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const v4u_t nib = h ? ((T.k[v] >> 4u) & kNib) : (T.k[v] & kNib);
                d[v][h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i_t, nib), Q.op[h],
                                                                v4i_t{nr[h], nr[h], nr[h], nr[h]}, 0, 0, 0);
            }
        after_qk();
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float4 k0 = *reinterpret_cast<const float4*>(&sm.kst[wave][m & 1][16 * v + 4 * g]);
            const float4 k1 = *reinterpret_cast<const float4*>(&sm.kst[wave][2 + (m & 1)][16 * v + 4 * g]);
            const float4 kb = *reinterpret_cast<const float4*>(&sm.kb[wave][16 * v + 4 * g]);
            const float a0[4] = {k0.x, k0.y, k0.z, k0.w};
            const float a1[4] = {k1.x, k1.y, k1.z, k1.w};
            const float b4[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float f = (float)d[v][0][r] * Q.sc[0] * a0[r];
                f = fmaf((float)d[v][1][r] * Q.sc[1], a1[r], f);
                s[v][r] = (f + dpp_f<kDppXor1>(f)) + b4[r];
            }
        }
    }
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
    // -8 in every f16 of a B operand: the products sum_t w_t * (-8) of a
    // block, added to both of its slices
    const v8h_t neg8 = {(_Float16)-8.0f, (_Float16)-8.0f, (_Float16)-8.0f, (_Float16)-8.0f,
                        (_Float16)-8.0f, (_Float16)-8.0f, (_Float16)-8.0f, (_Float16)-8.0f};
#pragma unroll
    for (int vp = 0; vp < 2; ++vp) {
        v8h_t A[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t wop[2][2];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int v = 2 * vp + q2;
                const float4 vv = *reinterpret_cast<const float4*>(&sm.vst[wave][b][16 * v + 4 * g]);
                const float w[4] = {p[v][0] * vv.x, p[v][1] * vv.y, p[v][2] * vv.z, p[v][3] * vv.w};
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    wop[q2][pr] = weight_part_f16x2(w[2 * pr], w[2 * pr + 1], part_mask);
                }
            }
            A[b] = __builtin_bit_cast(v8h_t, v4u_t{wop[0][0], wop[0][1], wop[1][0], wop[1][1]});
        }
        // codes of slice sl (d = 32(sl/2) + 2m + (sl&1): byte sl/2 of the
        // word, high nibble for odd sl) for tokens 2i, 2i+1 of the lane's 8
        // (token group 2vp + q/4, e = q%4) as one f16 pair: a code byte
        // 0..15 is c * 2^-9 as OCP fp8 e4m3, converted with scale 2^9
        uint32_t bw[8][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q0 = 2 * i, q1 = 2 * i + 1;
            const uint32_t wa = T.v[2 * vp + q0 / 4][q0 % 4], wb = T.v[2 * vp + q1 / 4][q1 % 4];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                // bytes [a(2hb), b(2hb), a(2hb+1), b(2hb+1)]
                const uint32_t x = __builtin_amdgcn_perm(wb, wa, hb ? 0x07030602u : 0x05010400u);
                const uint32_t xl = x & kNib, xh = (x >> 4) & kNib;
                bw[4 * hb + 0][i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xl, 512.0f, false));
                bw[4 * hb + 1][i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xh, 512.0f, false));
                bw[4 * hb + 2][i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xl, 512.0f, true));
                bw[4 * hb + 3][i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xh, 512.0f, true));
            }
        }
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            const v8h_t B = __builtin_bit_cast(v8h_t, v4u_t{bw[sl][0], bw[sl][1], bw[sl][2], bw[sl][3]});
            st.acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[sl >> 1], B, st.acc[sl], 0, 0, 0);
            st.acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[sl >> 1], neg8, st.acc[sl], 0, 0, 0);
        }
    }
}

// Fold the wave states and write one partial per query head (slice s of
// lane m holds d = 32(s/2) + 2m + (s&1)).
__device__ __forceinline__ void q40_write_partial(const DecodeArgs& a, QSmem40& sm, MState& st, int G, int b,
                                                  int kh, int c, int lane, int wave) {
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
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const float o0 = (st.acc[2 * kb][2 * hh] + st.acc[2 * kb][2 * hh + 1]) * unscale;
                const float o1 = (st.acc[2 * kb + 1][2 * hh] + st.acc[2 * kb + 1][2 * hh + 1]) * unscale;
                *reinterpret_cast<float2*>(&sm.acc[wave][H][32 * kb + 2 * m]) = make_float2(o0, o1);
            }
        }
    }
    lds_barrier();
    mcombine_write(a, sm, G, b, kh, c);
}

template <bool BS8>
__global__ __launch_bounds__(kWGThreads, 2) void kvq4_0_decode_kernel(DecodeArgs a) {
    __shared__ QSmem40 sm;
    // the arguments the prologue needs, read in one batch (as in the int8
    // chunk kernel)
    {
        const void* p0 = a.q;
        const void* p1 = a.r8.bt;
        const void* p2 = a.r8.lens;
        const void* p3 = a.k4;
        const void* p4 = a.ks;
        __asm__ volatile("" ::"s"(p0), "s"(p1), "s"(p2), "s"(p3), "s"(p4), "s"(a.nq), "s"(a.nkv), "s"(a.batch),
                         "s"(a.r8.max_chunks), "s"(a.tiles_per_wave), "s"(a.r8.max_blocks), "s"(a.r8.max_len),
                         "s"(a.log2_bs), "s"(a.r8.n_blocks));
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = a.nq / a.nkv;

    // work decode: the nkv workgroups of one (sequence, chunk) share an XCD,
    // pairs laid out at an odd stride
    const int nct = a.r8.max_chunks;
    const int wg = blockIdx.x;
    const int rest = wg >> 3;
    const int kh = rest % a.nkv;
    const int p = (rest / a.nkv) * 8 + (wg & 7);
    const int b = p / pair_stride(nct, a.batch);
    const int c = p - b * pair_stride(nct, a.batch);
    if (b >= a.batch || c >= nct) return;
    const int chunk_len = a.tiles_per_wave * kChunkUnit;
    const int c0 = c * chunk_len;
    const int32_t* btb = a.r8.bt + (size_t)b * a.r8.max_blocks;
    const int first = c0 + wave * kTile;
    int raw = mtile_raw(a.r8, btb, first, a.log2_bs, lane);
    const int L = effective_len(a.r8, b, a.log2_bs);
    if (c0 >= L) return;                                       // uniform per workgroup
    const int end = min(L, c0 + chunk_len);
    const int n_tiles = first < end ? (end - first + kChunkUnit - 1) / kChunkUnit : 1;

    const float4 qx = load_q4(a.q + ((size_t)b * a.nq + (size_t)kh * G) * kHD, G);
    const QLaneOff lo = q40_lane_offsets(lane);
    QTile A, B;
    qtile_issue<BS8>(a, raw, first, kh, lane, lo, A);
    raw = mtile_raw(a.r8, btb, first + kChunkUnit, a.log2_bs, lane);
    __asm__ volatile("" ::: "memory");

    quantize_q4(qx, G, sm.q);
    lds_barrier();
    const int g = lane >> 4;
    const int m = lane & 15;
    const MQuery Q = load_q_operand(sm.q, G, g, m);
    int nr[2];
    q40_block_bias(sm.q, G, m, nr);

    MState st;
    st.M = -INFINITY;
    st.S = 0.0f;
    st.E = 100;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) st.acc[sl] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};

    // double-buffered walk as in the int8 kernel
    int base = first;
    for (int k = 0;;) {
        if (k + 1 >= n_tiles) {
            qtile_compute(a, A, base, L, lane, wave, Q, nr, st, sm);
            break;
        }
        qtile_issue<BS8, kIssueKeys | kIssueSteps>(a, raw, base + kChunkUnit, kh, lane, lo, B);
        raw = mtile_raw(a.r8, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
        qtile_compute(a, A, base, L, lane, wave, Q, nr, st, sm, [&]() __attribute__((always_inline)) {
            qtile_issue<BS8, kIssueValues>(a, 0, base + kChunkUnit, kh, lane, lo, B);
        });
        base += kChunkUnit;
        ++k;
        if (k + 1 >= n_tiles) {
            qtile_compute(a, B, base, L, lane, wave, Q, nr, st, sm);
            break;
        }
        qtile_issue<BS8, kIssueKeys | kIssueSteps>(a, raw, base + kChunkUnit, kh, lane, lo, A);
        raw = mtile_raw(a.r8, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
        qtile_compute(a, B, base, L, lane, wave, Q, nr, st, sm, [&]() __attribute__((always_inline)) {
            qtile_issue<BS8, kIssueValues>(a, 0, base + kChunkUnit, kh, lane, lo, A);
        });
        base += kChunkUnit;
        ++k;
    }
    q40_write_partial(a, sm, st, G, b, kh, c, lane, wave);
}

template <bool BS8>
inline int launch_q40_bs(const DecodeArgs& a, int n_wg, hipStream_t s) {
    return launch((kvq4_0_decode_kernel<BS8>), dim3(n_wg), dim3(kWGThreads), s, a);
}

}  // namespace kvq

using namespace kvq;

extern "C" int kvq4_0_quantize_append(uint8_t* k_cache, uint8_t* v_cache, float* k_step, float* v_step,
                                      int n_blocks, int kv_bs, int nkv, int hd, const void* k_new,
                                      const void* v_new, int dtype, int n_tokens, const int32_t* slots,
                                      void* stream) {
    if (hd != kHD || !valid_block_size(kv_bs) || nkv < 1 || n_blocks < 1) return KVQ8_ESHAPE;
    if (n_tokens < 0 || dtype < KVQ8_F32 || dtype > KVQ8_F16) return KVQ8_EINVAL;
    if (n_tokens == 0) return KVQ8_OK;
    if (!k_cache || !v_cache || !k_step || !v_step || !k_new || !v_new || !slots) return KVQ8_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(k_step) || !aligned16(v_step))
        return KVQ8_EINVAL;
    const long n_rows = (long)n_tokens * nkv * 2;
    if (n_rows > 0x7FFFFFFFL - kQ40RowsPerBlock) return KVQ8_ESHAPE;
    const long n_slots = (long)n_blocks * kv_bs;
    // pool rows are 32-bit in the kernel: 2^32 rows would take over 320 GiB
    // of codes and steps
    if (n_slots * nkv > 0xFFFFFFFFL) return KVQ8_ESHAPE;
    const dim3 grid((unsigned)((n_rows + kQ40RowsPerBlock - 1) / kQ40RowsPerBlock)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
#define KVQ40_LAUNCH(DT)                                                                                    \
    launch(kvq4_0_quantize_append_kernel<DT>, grid, block, s, k_cache, v_cache, k_step, v_step,          \
           slot_cap(n_slots), make_divn(nkv), ilog2(kv_bs), k_new, v_new, (int)n_rows, slots)
    int st;
    if (dtype == KVQ8_F32) st = KVQ40_LAUNCH(KVQ8_F32);
    else if (dtype == KVQ8_BF16) st = KVQ40_LAUNCH(KVQ8_BF16);
    else st = KVQ40_LAUNCH(KVQ8_F16);
#undef KVQ40_LAUNCH
    return st;
}

extern "C" int kvq4_0_decode_chunk_tokens(int batch, int nkv, int max_ctx_len) {
    if (batch < 0 || nkv < 1 || max_ctx_len < 0) return 0;
    // two workgroups per CU: at least 512 of them, up to 2048 tokens each
    const long units = (long)batch * nkv;
    return default_tiles_per_wave(units, max_ctx_len, 8, 512) * kChunkUnit;
}

static int resolve_chunk40(int batch, int nkv, int max_ctx_len, int chunk) {
    if (chunk == 0) return kvq4_0_decode_chunk_tokens(batch, nkv, max_ctx_len);
    if (chunk < 0 || chunk % kChunkUnit != 0 || chunk > 64 * kChunkUnit) return -1;
    return chunk;
}

extern "C" size_t kvq4_0_decode_workspace_size(int batch, int nq, int nkv, int max_ctx_len, int chunk) {
    if (batch < 0 || nq < 1 || nkv < 1 || max_ctx_len < 0) return 0;
    const int ch = resolve_chunk40(batch, nkv, max_ctx_len, chunk);
    if (ch <= 0) return 0;
    return decode_workspace_bytes(batch, nq, (max_ctx_len + ch - 1) / ch);
}

extern "C" int kvq4_0_decode_attn(float* out, const float* q, int batch, int nq, const uint8_t* k_cache,
                                  const uint8_t* v_cache, const float* k_step, const float* v_step, int n_blocks,
                                  int kv_bs, int nkv, int hd, const int32_t* block_tables, int max_blocks_per_seq,
                                  const int32_t* ctx_lens, int max_ctx_len, float sm_scale, int chunk,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (!decode_shape_ok(batch, nq, nkv, hd, kv_bs) || n_blocks < 1 || max_blocks_per_seq < 1) return KVQ8_ESHAPE;
    if (!rows_fit_u32(n_blocks, kv_bs, nkv)) return KVQ8_ESHAPE;
    if (max_ctx_len < 0 || !score_scale_ok(sm_scale)) return KVQ8_EINVAL;
    const int ch = resolve_chunk40(batch, nkv, max_ctx_len, chunk);
    if (ch <= 0) return KVQ8_ESHAPE;
    if (batch == 0) return KVQ8_OK;
    if (!out || !q || !k_cache || !v_cache || !k_step || !v_step || !block_tables || !ctx_lens) return KVQ8_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_step) || !aligned16(v_step))
        return KVQ8_EINVAL;
    const size_t need = kvq4_0_decode_workspace_size(batch, nq, nkv, max_ctx_len, chunk);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KVQ8_EWORKSPACE;

    DecodeArgs a = {};
    a.q = q;
    a.k4 = k_cache;
    a.v4 = v_cache;
    a.ks = k_step;
    a.vs = v_step;
    a.r8 = Region{block_tables, ctx_lens, max_blocks_per_seq, max_ctx_len, n_blocks, (max_ctx_len + ch - 1) / ch};
    a.r4 = Region{nullptr, nullptr, 1, 0, 0, 0};
    a.nq = nq;
    a.nkv = nkv;
    a.log2_bs = ilog2(kv_bs);
    a.batch = batch;
    a.tiles_per_wave = ch / kChunkUnit;
    a.score_scale = score_scale(sm_scale) * kLog2e;
    bind_workspace(a, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int nct = n_chunks_total(a);
    if (nct > 0) {
        const long pairs = (long)a.batch * pair_stride(nct, a.batch);
        const long n_wg = (long)a.nkv * ((pairs + 7) / 8) * 8;
        if (n_wg > 0x7FFFFFFFL) return KVQ8_ESHAPE;
        const int st = a.log2_bs < 4 ? launch_q40_bs<true>(a, (int)n_wg, s) : launch_q40_bs<false>(a, (int)n_wg, s);
        if (st != KVQ8_OK) return st;
    }
    return launch_merge(a, out, s);
}
