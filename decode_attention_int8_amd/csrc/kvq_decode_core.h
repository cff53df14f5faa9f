// Split-K decode pipeline shared by the int8 and the int4-group entry points
// ([P3] Sec. 1-2 generalized to batches, paged blocks and grouped queries;
// int4 groups of [P4] Sec. 3.2).
//
// Work decomposition:
//   workgroup  = (sequence b, kv-head kh, context chunk c), kWaves waves;
//   wave tile  = 64 consecutive tokens of that kv-head;
//   lane       = token group tg = lane / 8 (one token per load row) and
//                segment j = lane % 8 (values 16j .. 16j+15 of the head row).
// An int8 load row therefore reads 8 whole 128-B rows (one per token group),
// an int4 load row 8 whole 64-B rows.
//
// Per tile the wave computes the int32 block dot products (v_dot4, DPP
// partner sums), scores in base-2 units (the score scale folds in log2 e),
// a tile max that rescales the running state only when it rises, and the
// value accumulation with float weights.  The workgroup merges its waves
// through LDS and writes one (M, S, acc[128]) partial per query head; the
// merge kernel combines the chunks and divides by the total sum
// ([P3] Sec. 2 seg. 3).
#pragma once

#include "kvq8.h"
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

constexpr int kWaves = 4;
constexpr int kWGThreads = kWaves * kWave;
constexpr int kMaxGroup = 8;
constexpr int kChunkUnit = kWaves * kTile;      // chunks are multiples of this
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kNib = 0x0F0F0F0Fu;

// One paged pool region: its block table and length clamp.
struct Region {
    const int32_t* bt;          // [batch][max_blocks]
    const int32_t* lens;        // [batch]
    int max_blocks;
    int max_len;
    int n_blocks;
    int max_chunks;             // ceil(max_len / chunk)
};

struct DecodeArgs {
    float* ws_acc;              // [batch][nq][n_chunks_total][128]
    float* ws_m;                // [batch][nq][n_chunks_total]
    float* ws_s;                // [batch][nq][n_chunks_total]
    const float* q;             // [batch][nq][128]
    // int8 pool
    const int8_t* kc;           // [n_blocks][bs][nkv][128]
    const int8_t* vc;
    const float* ks;            // [n_blocks][bs][nkv]
    const float* vs;
    // int4 pool
    const uint8_t* k4;          // [n_blocks4][bs][nkv][64]
    const uint8_t* v4;
    const uint16_t* k4s;        // [n_blocks4][bs][nkv][2] binary16
    const uint16_t* k4z;
    const uint16_t* v4s;
    const uint16_t* v4z;
    Region r8, r4;              // r4.max_chunks == 0 for the pure int8 path
    // fused write path: the token at position L-1 of every sequence
    const void* k_new;          // [batch][nkv][128], float32 / bf16 / f16
    const void* v_new;
    int8_t* kc_w;               // the int8 pool, written for that token
    int8_t* vc_w;
    float* ks_w;
    float* vs_w;
    int nq, nkv, log2_bs, batch;
    int tiles_per_wave;
    float score_scale;          // sm_scale * log2(e)
};

__device__ __host__ __forceinline__ int n_chunks_total(const DecodeArgs& a) {
    return a.r4.max_chunks + a.r8.max_chunks;
}

__device__ __forceinline__ int effective_len(const Region& r, int b, int log2_bs) {
    if (r.max_chunks == 0) return 0;
    long L = r.lens[b];
    const long cap = (long)r.max_blocks << log2_bs;
    if (L > r.max_len) L = r.max_len;
    if (L > cap) L = cap;
    return L < 0 ? 0 : (int)L;
}

// Block ids of the 8 rows of the tile at tile_base (row r holds tokens
// tile_base + 8r .. +7), or -1 for rows past L or with an id outside the
// pool.  One vector load (lane i reads row i % 8's table entry) and 8 lane
// reads put the ids in scalar registers after a single memory round trip.
// The table index is clamped to the row's capacity, not to L, so the load
// does not wait for the context length.
__device__ __forceinline__ int tile_block_raw(const Region& r, const int32_t* __restrict__ btb, int tile_base,
                                              int log2_bs, int lane) {
    const int t0 = tile_base + 8 * (lane & 7);
    return btb[min(t0 >> log2_bs, r.max_blocks - 1)];
}

__device__ __forceinline__ int tile_blocks_from(const Region& r, int raw, int tile_base, int L, int lane,
                                                int (&blk)[8]) {
    const int t0 = tile_base + 8 * (lane & 7);
    const int id = (t0 < L && raw >= 0 && raw < r.n_blocks) ? raw : -1;
#pragma unroll
    for (int i = 0; i < 8; ++i) blk[i] = __builtin_amdgcn_readlane(id, i);
    return id;
}

__device__ __forceinline__ int tile_blocks(const Region& r, const int32_t* __restrict__ btb, int tile_base, int L,
                                           int log2_bs, int lane, int (&blk)[8]) {
    return tile_blocks_from(r, tile_block_raw(r, btb, tile_base, log2_bs, lane), tile_base, L, lane, blk);
}

// Byte offset of row r's (token group 0, kv-head kh) entry in the pool, in
// units of one head row; wave-uniform.  An invalid row maps to 0 (slot 0 of
// the pool, always in bounds; its lanes are masked).
__device__ __forceinline__ size_t row_unit(int blk, int t0, int bs_mask, int nkv, int kh) {
    return blk >= 0 ? ((size_t)blk * (bs_mask + 1) + (t0 & bs_mask)) * nkv + kh : 0;
}

// ----------------------------------------------------------------------------
// running softmax state of one wave
// ----------------------------------------------------------------------------
template <int G>
struct WaveState {
    float m[G];        // running max (base-2 units), uniform across the wave
    float S[G];        // this lane's share of the running sum
    float acc[G][16];  // this lane's share of the value accumulator
    float accz[G];     // int4 zero-point correction (0 on the int8 path)

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = -INFINITY;
            S[h] = 0.0f;
            accz[h] = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[h][e] = 0.0f;
        }
    }

    // Raise the running max to the tile max of s[h][.] and return the
    // reference for this tile's exponentials.
    __device__ __forceinline__ float rebase(int h, const float (&s)[8]) {
        float mt = s[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) mt = fmaxf(mt, s[r]);
        mt = group8_max(mt);
        if (mt > m[h]) {
            const float sc = __builtin_amdgcn_exp2f(m[h] - mt);
            S[h] *= sc;
            accz[h] *= sc;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[h][e] *= sc;
            m[h] = mt;
        }
        // a tile whose tokens all sit in invalid blocks leaves m at -inf;
        // its weights must come out 0, not exp2(-inf - -inf)
        return (m[h] == -INFINITY) ? 0.0f : m[h];
    }
};

// ----------------------------------------------------------------------------
// int8 tile ([P3] Sec. 2 seg. 2)
//
// issue_*: the block ids of the tile's 8 rows are wave-uniform, so they come
// from scalar loads; all 16 vector loads of the rows then go out with no wait
// in between, and the caller can overlap them with other work.  Rows whose
// block is outside the pool are not read; lanes past the context end read
// their (in-bounds) slot and are masked at compute time.
// ----------------------------------------------------------------------------
struct TileQ8 {
    uint4 k[8], v[8];
    float ks[8], vs[8];
    bool valid[8];
    int ids;           // lane i holds row (i % 8)'s block id (-1 when invalid)
};

template <bool WITH_V>
__device__ __forceinline__ void issue_rows_q8(const DecodeArgs& a, const int (&blk)[8], int L, int kh, int tile_base,
                                              int tg, int j, TileQ8& T) {
    const int bs_mask = (1 << a.log2_bs) - 1;
    // lane part of every address: token group tg sits tg rows further on
    const uint32_t lane_row = (uint32_t)tg * a.nkv;
    size_t unit[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int t0 = tile_base + 8 * r;
        T.valid[r] = (blk[r] >= 0) && (t0 + tg < L);
        unit[r] = row_unit(blk[r], t0, bs_mask, a.nkv, kh);
    }
    // unconditional loads, all K rows before all V rows: the compiler can
    // count outstanding loads exactly, and scoring starts while V is in flight
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        T.k[r] = ldg16(a.kc + unit[r] * kHD + (lane_row * kHD + 16 * j));
        T.ks[r] = (a.ks + unit[r])[lane_row];
    }
    if constexpr (WITH_V) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            T.v[r] = ldg16(a.vc + unit[r] * kHD + (lane_row * kHD + 16 * j));
            T.vs[r] = (a.vs + unit[r])[lane_row];
        }
    }
}

template <bool WITH_V>
__device__ __forceinline__ void issue_tile_q8(const DecodeArgs& a, const int32_t* __restrict__ btb, int L, int kh,
                                              int tile_base, int tg, int j, TileQ8& T) {
    int blk[8];
    T.ids = tile_blocks(a.r8, btb, tile_base, L, a.log2_bs, __lane_id(), blk);
    issue_rows_q8<WITH_V>(a, blk, L, kh, tile_base, tg, j, T);
}

template <int G>
__device__ __forceinline__ void compute_tile_q8(const DecodeArgs& a, const TileQ8& T, const uint32_t (&qc)[G][4],
                                                const float (&qs)[G], WaveState<G>& st) {
    const uint4(&K8)[8] = T.k;
    const uint4(&V8)[8] = T.v;
    const float(&KS)[8] = T.ks;
    const float(&VS)[8] = T.vs;
    float w[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float s[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float f = block_scaled_sum(block_dot(qc[h], K8[r]), qs[h]);
            s[r] = T.valid[r] ? f * (KS[r] * a.score_scale) : -INFINITY;
        }
        const float mref = st.rebase(h, s);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float pr = __builtin_amdgcn_exp2f(s[r] - mref);
            st.S[h] += pr;
            // masked lanes may hold a stale slot's step: never let it in
            w[h][r] = T.valid[r] ? pr * VS[r] : 0.0f;
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t vw[4] = {V8[r].x, V8[r].y, V8[r].z, V8[r].w};
        float vf[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) vf[e] = sbyte_f(vw[e >> 2], e & 3);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.acc[h][e] = fmaf(w[h][r], vf[e], st.acc[h][e]);
    }
}

// ----------------------------------------------------------------------------
// int4 tile ([P4] Sec. 3.2 codes; integer scoring of the same Q8 codes)
//
// A lane's 16 values (8 packed bytes) all lie in group g = j / 4.  Packed
// byte k holds value 2k in its high nibble and 2k+1 in its low nibble, so
// (w >> 4) & 0x0F0F0F0F gives the even values and w & 0x0F0F0F0F the odd
// ones; the query codes are split the same way once per call.
// ----------------------------------------------------------------------------
struct Q4Query {
    uint32_t even[2];   // query codes 0,2,4,6 | 8,10,12,14 of the lane's 16
    uint32_t odd[2];    // query codes 1,3,5,7 | 9,11,13,15
    int rsum;           // R_b: sum of the query codes of the lane's block
};

__device__ __forceinline__ Q4Query split_q4(const uint32_t (&qc)[4]) {
    Q4Query o;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        // bytes of qc[2i] = q0 q1 q2 q3, qc[2i+1] = q4 q5 q6 q7 (little endian)
        o.even[i] = __builtin_amdgcn_perm(qc[2 * i + 1], qc[2 * i], 0x06040200u);
        o.odd[i] = __builtin_amdgcn_perm(qc[2 * i + 1], qc[2 * i], 0x07050301u);
    }
    int r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) r = __builtin_amdgcn_sdot4((int)qc[i], 0x01010101, r, false);
    o.rsum = r + dpp_i<kDppXor1>(r);
    return o;
}

__device__ __forceinline__ int block_dot_q4(const Q4Query& q, const uint2& k) {
    int d = __builtin_amdgcn_sdot4((int)q.even[0], (int)((k.x >> 4) & kNib), 0, false);
    d = __builtin_amdgcn_sdot4((int)q.odd[0], (int)(k.x & kNib), d, false);
    d = __builtin_amdgcn_sdot4((int)q.even[1], (int)((k.y >> 4) & kNib), d, false);
    d = __builtin_amdgcn_sdot4((int)q.odd[1], (int)(k.y & kNib), d, false);
    return d + dpp_i<kDppXor1>(d);
}

struct TileQ4 {
    uint2 k[8], v[8];
    float ks[8], kz[8], vs[8], vz[8];
    bool valid[8];
};

__device__ __forceinline__ void issue_tile_q4(const DecodeArgs& a, const int32_t* __restrict__ btb, int L, int kh,
                                              int tile_base, int tg, int j, TileQ4& T) {
    const int bs_mask = (1 << a.log2_bs) - 1;
    const int grp = j >> 2;
    const uint32_t lane_row = (uint32_t)tg * a.nkv;
    int blk[8];
    tile_blocks(a.r4, btb, tile_base, L, a.log2_bs, __lane_id(), blk);
    size_t unit[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int t0 = tile_base + 8 * r;
        T.valid[r] = (blk[r] >= 0) && (t0 + tg < L);
        unit[r] = row_unit(blk[r], t0, bs_mask, a.nkv, kh);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        T.k[r] = *reinterpret_cast<const uint2*>(a.k4 + unit[r] * (kHD / 2) + (lane_row * (kHD / 2) + 8 * j));
        T.ks[r] = half_bits_f((a.k4s + unit[r] * 2)[lane_row * 2 + grp]);
        T.kz[r] = half_bits_f((a.k4z + unit[r] * 2)[lane_row * 2 + grp]);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        T.v[r] = *reinterpret_cast<const uint2*>(a.v4 + unit[r] * (kHD / 2) + (lane_row * (kHD / 2) + 8 * j));
        T.vs[r] = half_bits_f((a.v4s + unit[r] * 2)[lane_row * 2 + grp]);
        T.vz[r] = half_bits_f((a.v4z + unit[r] * 2)[lane_row * 2 + grp]);
    }
}

template <int G>
__device__ __forceinline__ void compute_tile_q4(const DecodeArgs& a, const TileQ4& T, const Q4Query (&q4)[G],
                                                const float (&qs)[G], WaveState<G>& st) {
    float ws[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float s[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            // sum_b qsc_b * s_g * (P_b - z_g * R_b); z_g is an integer in [0, 15]
            const int term = block_dot_q4(q4[h], T.k[r]) - (T.valid[r] ? (int)T.kz[r] : 0) * q4[h].rsum;
            float f = (float)term * (qs[h] * T.ks[r]);
            f += dpp_f<kDppXor2>(f);
            f += dpp_f<kDppHalfMirror>(f);
            s[r] = T.valid[r] ? f * a.score_scale : -INFINITY;
        }
        const float mref = st.rebase(h, s);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float pr = __builtin_amdgcn_exp2f(s[r] - mref);
            st.S[h] += pr;
            ws[h][r] = T.valid[r] ? pr * T.vs[r] : 0.0f;
            st.accz[h] = fmaf(ws[h][r], T.valid[r] ? T.vz[r] : 0.0f, st.accz[h]);
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        float vf[16];
        const uint32_t lo[2] = {T.v[r].x & kNib, T.v[r].y & kNib};
        const uint32_t hi[2] = {(T.v[r].x >> 4) & kNib, (T.v[r].y >> 4) & kNib};
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                vf[8 * i + 2 * k] = (float)((hi[i] >> (8 * k)) & 0xFFu);
                vf[8 * i + 2 * k + 1] = (float)((lo[i] >> (8 * k)) & 0xFFu);
            }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.acc[h][e] = fmaf(ws[h][r], vf[e], st.acc[h][e]);
    }
}

// ----------------------------------------------------------------------------
// fused write path ([P2] Sec. 2): the new token's K / V rows, quantized by the
// 8 lanes of a token group (16 values per lane) with exactly the arithmetic of
// the write kernel (max |x|, step = max / 127, roundf(x / step), clamp +-127),
// so the codes are bit-identical to a separate kvq8_quantize_append.
// ----------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void load_new16(const void* base, size_t elem_off, float (&x)[16]) {
    if constexpr (DT == KVQ8_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 t = p[i];
            x[4 * i] = t.x;
            x[4 * i + 1] = t.y;
            x[4 * i + 2] = t.z;
            x[4 * i + 3] = t.w;
        }
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem_off);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 u = p[i];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (DT == KVQ8_BF16) {
                    x[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
                    x[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
                } else {
                    x[8 * i + 2 * k] = half_bits_f(w[k] & 0xFFFFu);
                    x[8 * i + 2 * k + 1] = half_bits_f(w[k] >> 16);
                }
            }
        }
    }
}

// Quantize a 128-value row held by an aligned 8-lane group, 16 values per
// lane: returns the lane's 16 codes (packed) and the row's step.
__device__ __forceinline__ void quantize_row8x16(const float (&x)[16], uint4& codes, float& d) {
#pragma clang fp contract(off)
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
    amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
    amax = fmaxf(amax, dpp_f<kDppHalfMirror>(amax));
    if (amax < 1e-6f) amax = 1.0f;
    d = amax / 127.0f;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float r = roundf(x[e] / d);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        w[e >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (e & 3));
    }
    codes = make_uint4(w[0], w[1], w[2], w[3]);
}

// ----------------------------------------------------------------------------
// workgroup merge and partial write
// ----------------------------------------------------------------------------
template <int G>
struct ReduceSmem {
    float acc[kWaves][4][G][kHD];
    float m[kWaves][G];
    float s[kWaves][G];
};

template <int G>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, ReduceSmem<G>& sm, WaveState<G>& st, int b,
                                              int kh, int c, int lane, int wave) {
    const int tg = lane >> 3;
    const int j = lane & 7;
    // Token groups tg and tg^1 fold with one DPP step; the even token groups
    // of every wave then meet in LDS.
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float v = st.acc[h][e] - st.accz[h];
            st.acc[h][e] = v + dpp_f<kDppRowRor8>(v);
        }
        const float tot = group8_sum(st.S[h]);
        if (lane == 0) {
            sm.m[wave][h] = st.m[h];
            sm.s[wave][h] = tot;
        }
    }
    if ((tg & 1) == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float4* dst = reinterpret_cast<float4*>(&sm.acc[wave][tg >> 1][h][16 * j]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[e] = make_float4(st.acc[h][4 * e], st.acc[h][4 * e + 1], st.acc[h][4 * e + 2],
                                     st.acc[h][4 * e + 3]);
        }
    }
    __syncthreads();
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
                const float part = (sm.acc[wv][0][h][d] + sm.acc[wv][1][h][d]) +
                                   (sm.acc[wv][2][h][d] + sm.acc[wv][3][h][d]);
                tot = fmaf(part, f, tot);
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

// ----------------------------------------------------------------------------
// the chunk kernel.  Chunks [0, r4.max_chunks) cover the int4 region, the
// rest the int8 region.
// ----------------------------------------------------------------------------
// Walk this wave's tiles of the chunk: first, first + kWaves*64, ... < end.
// The caller has already issued the first tile (always, so that no load
// sits behind a branch and the compiler can count outstanding loads).
template <class Tile, class Issue, class Compute>
__device__ __forceinline__ void walk_tiles(int c0, int first, int end, Tile& A, Issue issue, Compute compute) {
    for (int base = first; base < end;) {
        compute(base, A);
        base += kWaves * kTile;
        if (base < end) issue(base, A);
    }
}

template <int G>
__global__ __launch_bounds__(kWGThreads) void kvq4_decode_chunk_kernel(DecodeArgs a) {
    __shared__ ReduceSmem<G> sm;
    __shared__ QSmem qsm;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int tg = lane >> 3;
    const int j = lane & 7;

    // Work decode.  Workgroups are dealt to the 8 XCDs in turn; the nkv
    // workgroups of one (sequence, chunk) land on the same XCD, so the step
    // lines they share (token-major layout) stay in that XCD's L2.
    const int nct = n_chunks_total(a);
    const int wg = blockIdx.x;
    const int xcd = wg & 7;
    const int rest = wg >> 3;
    const int kh = rest % a.nkv;
    const int p = (rest / a.nkv) * 8 + xcd;
    const int b = p / nct;
    const int c = p - b * nct;
    if (b >= a.batch) return;
    const bool int4_region = c < a.r4.max_chunks;
    const Region& reg = int4_region ? a.r4 : a.r8;
    const int cr = int4_region ? c : c - a.r4.max_chunks;
    const int chunk_len = a.tiles_per_wave * kChunkUnit;
    const int c0 = cr * chunk_len;
    const int32_t* btb = reg.bt + (size_t)b * reg.max_blocks;
    // the query loads and the first tile's table entries go out together
    // with the length load
    const float4 qx = load_q4(a.q + ((size_t)b * a.nq + (size_t)kh * G) * kHD, G);
    const int raw0 = tile_block_raw(reg, btb, c0 + wave * kTile, a.log2_bs, lane);
    const int L = effective_len(reg, b, a.log2_bs);
    if (c0 >= L) return;                                   // uniform per workgroup
    const int end = min(L, c0 + chunk_len);
    const int first = c0 + wave * kTile;

    WaveState<G> st;
    st.init();
    uint32_t qc[G][4];
    float qs[G];
    // [P3] Sec. 2 seg. 1: the group's query heads are quantized once per
    // workgroup (into LDS); lane segment j takes codes 16j .. 16j+15 and the
    // scale of block j/2.
    auto query_codes = [&]() __attribute__((always_inline)) {
        quantize_q4(qx, G, qsm);
        lds_barrier();
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint4 w = *reinterpret_cast<const uint4*>(&qsm.qc[h][4 * j]);
            qc[h][0] = w.x;
            qc[h][1] = w.y;
            qc[h][2] = w.z;
            qc[h][3] = w.w;
            qs[h] = qsm.qs[h][j >> 1];
        }
    };

    // A wave without a tile (first >= L) still issues one: every row is then
    // invalid, reads slot 0 of the pool and is discarded.
    if (int4_region) {
        TileQ4 A;
        issue_tile_q4(a, btb, L, kh, first, tg, j, A);
        query_codes();
        Q4Query q4[G];
#pragma unroll
        for (int h = 0; h < G; ++h) q4[h] = split_q4(qc[h]);
        walk_tiles(
            c0, first, end, A, [&](int base, TileQ4& T) { issue_tile_q4(a, btb, L, kh, base, tg, j, T); },
            [&](int, const TileQ4& T) { compute_tile_q4<G>(a, T, q4, qs, st); });
    } else {
        TileQ8 A;
        int blk[8];
        A.ids = tile_blocks_from(a.r8, raw0, first, L, lane, blk);
        issue_rows_q8<true>(a, blk, L, kh, first, tg, j, A);
        query_codes();
        walk_tiles(
            c0, first, end, A, [&](int base, TileQ8& T) { issue_tile_q8<true>(a, btb, L, kh, base, tg, j, T); },
            [&](int, const TileQ8& T) { compute_tile_q8<G>(a, T, qc, qs, st); });
    }
    write_partial<G>(a, sm, st, b, kh, c, lane, wave);
}

// Merge the chunk partials of one (sequence, query head) and normalize
// ([P3] Sec. 2 seg. 3 across chunks): M = max_c M_c, S = sum_c S_c 2^(M_c-M),
// out = sum_c acc_c 2^(M_c-M) / S.  256 threads: thread (part, d) owns output
// dimension d for half of the chunks; the two halves meet in LDS.  Chunks are
// read in batches of kMergeBatch with every load of a batch in flight (so up
// to 2 * kMergeBatch chunks cost one memory round trip); the loads do not wait
// for the context lengths (chunks past them are masked afterwards), and
// batches are combined with a running maximum.
constexpr int kMergeBatch = 16;
constexpr int kMergeThreads = 2 * kHD;

__global__ __launch_bounds__(kMergeThreads) void kvq_merge_kernel(float* __restrict__ out, DecodeArgs a) {
    __shared__ float other[kHD + 2];
    const int bh = blockIdx.x;
    const int b = bh / a.nq;
    const int d = threadIdx.x & (kHD - 1);
    const int part = __builtin_amdgcn_readfirstlane(threadIdx.x / kHD);
    const int chunk_len = a.tiles_per_wave * kChunkUnit;
    const int nct = n_chunks_total(a);
    const int half = (nct + 1) / 2;
    const int cbeg = part * half;
    const int cend = min(nct, cbeg + half);
    const int base8 = a.r4.max_chunks;
    const float* mm = a.ws_m + (size_t)bh * nct;
    const float* ss = a.ws_s + (size_t)bh * nct;
    const float* aa = a.ws_acc + (size_t)bh * nct * kHD + d;
    const int n4 = (effective_len(a.r4, b, a.log2_bs) + chunk_len - 1) / chunk_len;
    const int n8 = (effective_len(a.r8, b, a.log2_bs) + chunk_len - 1) / chunk_len;
    float M = -INFINITY, S = 0.0f, acc = 0.0f;
    for (int c0 = cbeg; c0 < cend; c0 += kMergeBatch) {
        float mv[kMergeBatch], sv[kMergeBatch], av[kMergeBatch];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const int cc = min(c0 + k, cend - 1);
            mv[k] = mm[cc];
            sv[k] = ss[cc];
            av[k] = aa[(size_t)cc * kHD];
        }
        float bm = -INFINITY;
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const int c = c0 + k;
            const bool live = c < cend && (c < n4 || (c >= base8 && c < base8 + n8));
            mv[k] = live ? mv[k] : -INFINITY;
            sv[k] = live ? sv[k] : 0.0f;   // a chunk never written may hold anything
            av[k] = live ? av[k] : 0.0f;
            bm = fmaxf(bm, mv[k]);
        }
        if (bm > M) {
            const float f = __builtin_amdgcn_exp2f(M - bm);
            S *= f;
            acc *= f;
            M = bm;
        }
        if (M == -INFINITY) continue;
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const float f = __builtin_amdgcn_exp2f(mv[k] - M);
            S = fmaf(sv[k], f, S);
            acc = fmaf(av[k], f, acc);
        }
    }
    if (part == 1) {
        other[d] = acc;
        if (d == 0) {
            other[kHD] = M;
            other[kHD + 1] = S;
        }
    }
    __syncthreads();
    if (part == 0) {
        const float M1 = other[kHD], S1 = other[kHD + 1], A1 = other[d];
        const float Mt = fmaxf(M, M1);
        float res = 0.0f;
        if (Mt != -INFINITY) {
            const float f0 = __builtin_amdgcn_exp2f(M - Mt), f1 = __builtin_amdgcn_exp2f(M1 - Mt);
            res = fmaf(acc, f0, A1 * f1) / fmaf(S, f0, S1 * f1);
        }
        out[(size_t)bh * kHD + d] = res;
    }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

// Tokens per chunk: the largest power-of-two multiple of 256 that still gives
// at least 256 workgroups (one per CU), capped at 2048 for one or two
// sequences and at 1024 for batches (whose lengths vary, so shorter
// workgroups balance better).  `units` = sequences x kv-heads, `max_len` the
// longest region.
inline int default_tiles_per_wave(long batch, long units, long max_len) {
    const int cap = batch <= 2 ? 8 : 4;
    int tpw = 1;
    while (tpw < cap) {
        const long next = (long)kChunkUnit * tpw * 2;
        if (units * ((max_len + next - 1) / next) < 256) break;
        tpw *= 2;
    }
    return tpw;
}

inline bool decode_shape_ok(int batch, int nq, int nkv, int hd, int kv_bs) {
    if (hd != kHD || !valid_block_size(kv_bs) || nkv < 1 || nq < 1 || batch < 0) return false;
    if (nq % nkv != 0) return false;
    const int g = nq / nkv;
    return g >= 1 && g <= kMaxGroup;
}

// The int8 decode kernel indexes cache rows (one per slot and kv-head) with
// 32-bit integers.
inline bool rows_fit_u32(int n_blocks, int kv_bs, int nkv) {
    return (unsigned long long)n_blocks * (unsigned long long)kv_bs * (unsigned long long)nkv <= 0xFFFFFFFFull;
}

inline size_t decode_workspace_bytes(int batch, int nq, int n_chunks_total) {
    const size_t n = (size_t)batch * nq * n_chunks_total;
    return round_up(n * kHD * sizeof(float), 256) + 2 * round_up(n * sizeof(float), 256);
}

inline void bind_workspace(DecodeArgs& a, void* workspace) {
    const size_t n = (size_t)a.batch * a.nq * n_chunks_total(a);
    char* ws = static_cast<char*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(ws);
    a.ws_m = reinterpret_cast<float*>(ws + round_up(n * kHD * sizeof(float), 256));
    a.ws_s = reinterpret_cast<float*>(ws + round_up(n * kHD * sizeof(float), 256) + round_up(n * sizeof(float), 256));
}

template <int G>
inline void launch_chunks4(const DecodeArgs& a, int n_wg, hipStream_t s) {
    hipLaunchKernelGGL(kvq4_decode_chunk_kernel<G>, dim3(n_wg), dim3(kWGThreads), 0, s, a);
}

#define KVQ_DISPATCH_G(g, fn, ...)           \
    switch (g) {                             \
        case 1: fn<1>(__VA_ARGS__); break;   \
        case 2: fn<2>(__VA_ARGS__); break;   \
        case 3: fn<3>(__VA_ARGS__); break;   \
        case 4: fn<4>(__VA_ARGS__); break;   \
        case 5: fn<5>(__VA_ARGS__); break;   \
        case 6: fn<6>(__VA_ARGS__); break;   \
        case 7: fn<7>(__VA_ARGS__); break;   \
        default: fn<8>(__VA_ARGS__); break;  \
    }


}  // namespace kvq
