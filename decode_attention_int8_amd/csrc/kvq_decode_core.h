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

// Block id holding tokens t0 .. t0+7 (t0 a multiple of 8), or -1.
__device__ __forceinline__ int row_block(const Region& r, const int32_t* btb, int t0, int L, int log2_bs) {
    const int blk = (t0 < L) ? btb[t0 >> log2_bs] : -1;
    return (blk >= 0 && blk < r.n_blocks) ? blk : -1;
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
// ----------------------------------------------------------------------------
template <bool WITH_V>
__device__ __forceinline__ void load_tile_q8(const DecodeArgs& a, const int32_t* __restrict__ btb, int L, int kh,
                                             int tile_base, int tg, int j, uint4 (&kr)[8], uint4 (&vr)[8],
                                             float (&ksr)[8], float (&vsr)[8], bool (&valid)[8]) {
    const int bs_mask = (1 << a.log2_bs) - 1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int t0 = tile_base + 8 * r;
        const int t = t0 + tg;
        const int blk = row_block(a.r8, btb, t0, L, a.log2_bs);
        valid[r] = (t < L) && (blk >= 0);
        kr[r] = make_uint4(0, 0, 0, 0);
        vr[r] = make_uint4(0, 0, 0, 0);
        ksr[r] = 0.0f;
        vsr[r] = 0.0f;
        if (valid[r]) {
            const size_t row = ((size_t)blk * (bs_mask + 1) + (t & bs_mask)) * a.nkv + kh;
            kr[r] = ldg16(a.kc + row * kHD + 16 * j);
            ksr[r] = a.ks[row];
            if constexpr (WITH_V) {
                vr[r] = ldg16(a.vc + row * kHD + 16 * j);
                vsr[r] = a.vs[row];
            }
        }
    }
}

template <int G>
__device__ __forceinline__ void tile_q8(const DecodeArgs& a, const int32_t* __restrict__ btb, int L, int kh,
                                        int tile_base, int tg, int j, const uint32_t (&qc)[G][4],
                                        const float (&qs)[G], WaveState<G>& st) {
    uint4 kr[8], vr[8];
    float ksr[8], vsr[8];
    bool valid[8];
    load_tile_q8<true>(a, btb, L, kh, tile_base, tg, j, kr, vr, ksr, vsr, valid);

    float w[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float s[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float f = block_scaled_sum(block_dot(qc[h], kr[r]), qs[h]);
            s[r] = valid[r] ? f * (ksr[r] * a.score_scale) : -INFINITY;
        }
        const float mref = st.rebase(h, s);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float pr = __builtin_amdgcn_exp2f(s[r] - mref);
            st.S[h] += pr;
            w[h][r] = pr * vsr[r];
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t vw[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
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

template <int G>
__device__ __forceinline__ void tile_q4(const DecodeArgs& a, const int32_t* __restrict__ btb, int L, int kh,
                                        int tile_base, int tg, int j, const Q4Query (&q4)[G],
                                        const float (&qs)[G], WaveState<G>& st) {
    const int bs_mask = (1 << a.log2_bs) - 1;
    const int grp = j >> 2;
    uint2 kr[8], vr[8];
    float ksc[8], kz[8], vsc[8], vz[8];
    bool valid[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int t0 = tile_base + 8 * r;
        const int t = t0 + tg;
        const int blk = row_block(a.r4, btb, t0, L, a.log2_bs);
        valid[r] = (t < L) && (blk >= 0);
        kr[r] = make_uint2(0, 0);
        vr[r] = make_uint2(0, 0);
        ksc[r] = kz[r] = vsc[r] = vz[r] = 0.0f;
        if (valid[r]) {
            const size_t row = ((size_t)blk * (bs_mask + 1) + (t & bs_mask)) * a.nkv + kh;
            kr[r] = *reinterpret_cast<const uint2*>(a.k4 + row * (kHD / 2) + 8 * j);
            vr[r] = *reinterpret_cast<const uint2*>(a.v4 + row * (kHD / 2) + 8 * j);
            ksc[r] = half_bits_f(a.k4s[row * 2 + grp]);
            kz[r] = half_bits_f(a.k4z[row * 2 + grp]);
            vsc[r] = half_bits_f(a.v4s[row * 2 + grp]);
            vz[r] = half_bits_f(a.v4z[row * 2 + grp]);
        }
    }

    float ws[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float s[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            // sum_b qsc_b * s_g * (P_b - z_g * R_b); z_g is an integer in [0, 15]
            const int term = block_dot_q4(q4[h], kr[r]) - (int)kz[r] * q4[h].rsum;
            float f = (float)term * (qs[h] * ksc[r]);
            f += dpp_f<kDppXor2>(f);
            f += dpp_f<kDppHalfMirror>(f);
            s[r] = valid[r] ? f * a.score_scale : -INFINITY;
        }
        const float mref = st.rebase(h, s);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float pr = __builtin_amdgcn_exp2f(s[r] - mref);
            st.S[h] += pr;
            ws[h][r] = pr * vsc[r];
            st.accz[h] = fmaf(ws[h][r], vz[r], st.accz[h]);
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        float vf[16];
        const uint32_t lo[2] = {vr[r].x & kNib, vr[r].y & kNib};
        const uint32_t hi[2] = {(vr[r].x >> 4) & kNib, (vr[r].y >> 4) & kNib};
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
template <int G>
__global__ __launch_bounds__(kWGThreads) void kvq_decode_chunk_kernel(DecodeArgs a) {
    __shared__ ReduceSmem<G> sm;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
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
    const int L = effective_len(reg, b, a.log2_bs);
    const int chunk_len = a.tiles_per_wave * kChunkUnit;
    const int c0 = cr * chunk_len;
    if (c0 >= L) return;                                   // uniform per workgroup

    // [P3] Sec. 2 seg. 1: the group's query heads are quantized once.
    uint32_t qc[G][4];
    float qs[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
        quantize_q_segment(a.q + ((size_t)b * a.nq + (size_t)kh * G + h) * kHD, j, qc[h], qs[h]);

    WaveState<G> st;
    st.init();
    const int32_t* btb = reg.bt + (size_t)b * reg.max_blocks;
    if (int4_region) {
        Q4Query q4[G];
#pragma unroll
        for (int h = 0; h < G; ++h) q4[h] = split_q4(qc[h]);
        for (int tt = 0; tt < a.tiles_per_wave; ++tt) {
            const int tile_base = c0 + (tt * kWaves + wave) * kTile;
            if (tile_base >= L) break;                     // uniform per wave
            tile_q4<G>(a, btb, L, kh, tile_base, tg, j, q4, qs, st);
        }
    } else {
        for (int tt = 0; tt < a.tiles_per_wave; ++tt) {
            const int tile_base = c0 + (tt * kWaves + wave) * kTile;
            if (tile_base >= L) break;                     // uniform per wave
            tile_q8<G>(a, btb, L, kh, tile_base, tg, j, qc, qs, st);
        }
    }
    write_partial<G>(a, sm, st, b, kh, c, lane, wave);
}

// Merge the chunk partials of one (sequence, query head) and normalize.
__global__ __launch_bounds__(kHD) void kvq_merge_kernel(float* __restrict__ out, DecodeArgs a) {
    const int bh = blockIdx.x;
    const int b = bh / a.nq;
    const int d = threadIdx.x;
    const int chunk_len = a.tiles_per_wave * kChunkUnit;
    const int nct = n_chunks_total(a);
    const int n4 = (effective_len(a.r4, b, a.log2_bs) + chunk_len - 1) / chunk_len;
    const int n8 = (effective_len(a.r8, b, a.log2_bs) + chunk_len - 1) / chunk_len;
    const float* mm = a.ws_m + (size_t)bh * nct;
    const float* ss = a.ws_s + (size_t)bh * nct;
    const float* aa = a.ws_acc + (size_t)bh * nct * kHD + d;
    float M = -INFINITY;
    for (int c = 0; c < n4; ++c) M = fmaxf(M, mm[c]);
    for (int c = a.r4.max_chunks; c < a.r4.max_chunks + n8; ++c) M = fmaxf(M, mm[c]);
    float res = 0.0f;
    if (M != -INFINITY) {
        float S = 0.0f, acc = 0.0f;
        for (int c = 0; c < n4; ++c) {
            const float f = __builtin_amdgcn_exp2f(mm[c] - M);
            S = fmaf(ss[c], f, S);
            acc = fmaf(aa[(size_t)c * kHD], f, acc);
        }
        for (int c = a.r4.max_chunks; c < a.r4.max_chunks + n8; ++c) {
            const float f = __builtin_amdgcn_exp2f(mm[c] - M);
            S = fmaf(ss[c], f, S);
            acc = fmaf(aa[(size_t)c * kHD], f, acc);
        }
        res = acc / S;
    }
    out[(size_t)bh * kHD + d] = res;
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

// Smallest chunk that still gives ~1024 workgroups (four per CU), capped at
// 8 tiles per wave.  `units` = sequences x kv-heads, `max_len` the longest
// region.
inline int default_tiles_per_wave(long units, long max_len) {
    int tpw = 1;
    while (tpw < 8) {
        const long next = (long)kChunkUnit * tpw * 2;
        if (units * ((max_len + next - 1) / next) < 1024) break;
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
inline void launch_chunks(const DecodeArgs& a, int n_wg, hipStream_t s) {
    hipLaunchKernelGGL(kvq_decode_chunk_kernel<G>, dim3(n_wg), dim3(kWGThreads), 0, s, a);
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

// Enqueue the chunk kernel (if there is any context) and the merge kernel.
inline int launch_decode(const DecodeArgs& a, float* out, hipStream_t s) {
    const int nct = n_chunks_total(a);
    if (nct > 0) {
        const long pairs = (long)a.batch * nct;
        const long n_wg = (long)a.nkv * ((pairs + 7) / 8) * 8;
        if (n_wg > 0x7FFFFFFFL) return KVQ8_ESHAPE;
        KVQ_DISPATCH_G(a.nq / a.nkv, launch_chunks, a, (int)n_wg, s);
    }
    hipLaunchKernelGGL(kvq_merge_kernel, dim3(a.batch * a.nq), dim3(kHD), 0, s, out, a);
    return launch_status();
}

}  // namespace kvq
