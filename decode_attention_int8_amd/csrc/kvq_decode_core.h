// Shared parts of the split-K decode ([P3] Sec. 1-2 generalized to batches,
// paged blocks and grouped queries; int4 groups of [P4] Sec. 3.2): the
// argument block, the fused write path's quantizer, the merge kernel and the
// host-side sizing.
//
// Work decomposition: workgroup = (sequence b, kv-head kh, context chunk c),
// kWaves waves; wave tile = 64 consecutive tokens of that kv-head.  Each
// workgroup writes one (M, S, acc[128]) partial per query head; the merge
// kernel combines the chunks and divides by the total sum ([P3] Sec. 2
// seg. 3).
#pragma once

#include <type_traits>

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

// The banded cache adds the 2-bit pool, in an argument block of its own so
// that the int8, int4 and Q4_0 kernels keep theirs.  Chunk index space:
// [0, r2) 2-bit, [r2, r2 + r4) int4, then int8.
struct BandArgs : DecodeArgs {
    const uint8_t* k2;          // [n_blocks2][bs][nkv][32]
    const uint8_t* v2;
    const uint16_t* k2s;        // [n_blocks2][bs][nkv][2] binary16
    const uint16_t* k2z;
    const uint16_t* v2s;
    const uint16_t* v2z;
    Region r2;
};

__device__ __host__ __forceinline__ int n_chunks_total(const DecodeArgs& a) {
    return a.r4.max_chunks + a.r8.max_chunks;
}

__device__ __host__ __forceinline__ int n_chunks_total(const BandArgs& a) {
    return a.r2.max_chunks + a.r4.max_chunks + a.r8.max_chunks;
}

template <class Args>
inline constexpr bool kBanded = std::is_same_v<Args, BandArgs>;

// Workgroups are dealt to the 8 XCDs round-robin, and the grid is laid out so
// that pair p = (sequence, chunk) of every kv-head sits on XCD p % 8, at
// p = sequence * stride + chunk.  With several sequences of different lengths
// the low chunks are live for all of them and the high ones only for the
// long ones; an even stride (a chunk count that is a multiple of 8) would put
// chunk c of every sequence on XCD c % 8 and load the low XCDs with most of
// the work.  An odd stride walks every chunk index over all 8 XCDs.  One
// sequence needs no padding (its chunks already cycle over the XCDs).
__device__ __host__ __forceinline__ int pair_stride(int n_chunks, int batch) {
    return batch > 1 ? (n_chunks | 1) : n_chunks;
}

// A sequence's length clamped to [0, min(max_len, max_blocks * kv_bs)]:
// from its raw value, and from the lengths array.
__device__ __forceinline__ int clamp_len(const Region& r, int raw, int log2_bs) {
    long L = raw;
    const long cap = (long)r.max_blocks << log2_bs;
    if (L > r.max_len) L = r.max_len;
    if (L > cap) L = cap;
    return L < 0 ? 0 : (int)L;
}

__device__ __forceinline__ int effective_len(const Region& r, int b, int log2_bs) {
    if (r.max_chunks == 0) return 0;
    return clamp_len(r, r.lens[b], log2_bs);
}

// The same, also giving the length as read (0 for an empty region).
__device__ __forceinline__ int effective_len(const Region& r, int b, int log2_bs, int& raw) {
    raw = 0;
    if (r.max_chunks == 0) return 0;
    raw = r.lens[b];
    return clamp_len(r, raw, log2_bs);
}

// Dense work list of a batch decode over one int8 region (at most 64
// sequences).  The live (sequence, chunk) pairs are numbered so that every
// sequence's full chunks come first (sequence by sequence) and the partial
// last chunks after them, longest first; pair j then goes to XCD j % 8 like
// any pair index.  Each XCD so gets every eighth pair of that order (the
// same work to within a chunk), the workgroups past the last live pair are
// all at the end of the grid, and the last workgroups dispatched are the
// shortest.  Every lane computes it from the lengths (lane i reads sequence
// i's); the results are wave-uniform.  Returns false for j past the last pair.
constexpr int kDenseMaxBatch = kWave;

struct DenseItem {
    int b, c, L, lraw;
};

__device__ __forceinline__ bool dense_item(const Region& r, int batch, int log2_bs, int chunk_len, int j, int lane,
                                           DenseItem& it) {
    int raw = 0, Li = 0;
    if (lane < batch) {
        raw = r.lens[lane];
        Li = clamp_len(r, raw, log2_bs);
    }
    const int full = Li / chunk_len;
    const int rem = Li - full * chunk_len;
    int pre = full;                                        // inclusive prefix sum over lanes
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(pre, d);
        if (lane >= d) pre += o;
    }
    const int n_full = __builtin_amdgcn_readlane(pre, kWave - 1);
    int b, c;
    if (j < n_full) {
        b = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(pre > j));
        c = j - (__builtin_amdgcn_readlane(pre, b) - __builtin_amdgcn_readlane(full, b));
    } else {
        const int want = j - n_full;
        if (want >= (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(rem > 0))) return false;
        // rank among the partial chunks: longer first, equal lengths by sequence
        int rank = 0;
        for (int k = 0; k < batch; ++k) {
            const int rk = __builtin_amdgcn_readlane(rem, k);
            rank += (rk > rem || (rk == rem && k < lane)) ? 1 : 0;
        }
        b = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(rem > 0 && rank == want));
        c = __builtin_amdgcn_readlane(full, b);
    }
    it.b = b;
    it.c = c;
    it.L = __builtin_amdgcn_readlane(Li, b);
    it.lraw = __builtin_amdgcn_readlane(raw, b);
    return true;
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

// The new token's rows for the fused write path: lanes 0-31 hold 4 values
// of the K row, lanes 32-63 4 values of the V row (elements 4 (lane % 32) ..).
template <int DT>
__device__ __forceinline__ void load_new4(const void* base, size_t elem_off, float (&x)[4]) {
    if constexpr (DT == KVQ8_F32) {
        const float4 t = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
        x[0] = t.x;
        x[1] = t.y;
        x[2] = t.z;
        x[3] = t.w;
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + elem_off);
        const uint32_t w[2] = {u.x, u.y};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if constexpr (DT == KVQ8_BF16) {
                x[2 * k] = __uint_as_float(w[k] << 16);
                x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
            } else {
                x[2 * k] = half_bits_f(w[k] & 0xFFFFu);
                x[2 * k + 1] = half_bits_f(w[k] >> 16);
            }
        }
    }
}

// Quantize a 128-value row held by an aligned 32-lane half of the wave, 4
// values per lane (the int8 write path's rule, the maximum over 32 lanes):
// returns the lane's 4 codes (one word) and the row's step.
__device__ __forceinline__ void quantize_row32x4(const float (&x)[4], uint32_t& codes, float& d) {
#pragma clang fp contract(off)
    float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
    amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
    amax = fmaxf(amax, dpp_f<kDppHalfMirror>(amax));
    amax = fmaxf(amax, dpp_f<kDppRowRor8>(amax));
    amax = fmaxf(amax, swz_xor16(amax));
    if (amax < 1e-6f) amax = 1.0f;
    d = amax / 127.0f;
    const float rd = __builtin_amdgcn_rcpf(d);
    uint32_t w = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // roundf(x / d), the quotient computed only near a half-integer
        // (|x / d| <= 127)
        const float q = x[e] * rd;
        float r = rintf(q);
        if (near_half_small(q, r)) r = roundf(x[e] / d);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        w |= ((uint32_t)(int)r & 0xFFu) << (8 * e);
    }
    codes = w;
}

// Merge the chunk partials of one (sequence, query head) and normalize
// ([P3] Sec. 2 seg. 3 across chunks): M = max_c M_c, S = sum_c S_c 2^(M_c-M),
// out = sum_c acc_c 2^(M_c-M) / S.  PARTS x 128 threads: thread (part, d)
// owns output dimension d for a contiguous share of the chunks; the parts
// meet in LDS.  Chunks are read in batches of kMergeBatch with every load of a
// batch in flight (so up to PARTS * kMergeBatch chunks cost one memory round
// trip), and batches are combined with a running maximum.  With LIVE (one
// int8 region, several sequences of different lengths) a part reads only the
// chunks below its sequence's length, after loading that length; otherwise the
// loads do not wait for the lengths and chunks past them are masked afterwards.
constexpr int kMergeBatch = 16;
constexpr int kMergeThreads = 2 * kHD;          // PARTS = 2
constexpr int kMergeThreadsWide = 8 * kHD;      // PARTS = 8, for more than 32 chunks

template <int PARTS, bool LIVE = false, class Args = DecodeArgs, int BATCH = kMergeBatch>
__global__ __launch_bounds__(PARTS * kHD) void kvq_merge_kernel(float* __restrict__ out, Args a) {
    constexpr bool HAS2 = kBanded<Args>;
    __shared__ float other[PARTS][kHD + 2];
    const int bh = blockIdx.x;
    const int b = bh / a.nq;
    const int d = threadIdx.x & (kHD - 1);
    const int part = __builtin_amdgcn_readfirstlane(threadIdx.x / kHD);
    const int chunk_len = a.tiles_per_wave * kChunkUnit;
    const int nct = n_chunks_total(a);
    const int share = (nct + PARTS - 1) / PARTS;
    const int cbeg = part * share;
    int cend = min(nct, cbeg + share);
    int base4 = 0, n2 = 0;
    if constexpr (HAS2) base4 = a.r2.max_chunks;
    const int base8 = base4 + a.r4.max_chunks;
    const float* mm = a.ws_m + (size_t)bh * nct;
    const float* ss = a.ws_s + (size_t)bh * nct;
    const float* aa = a.ws_acc + (size_t)bh * nct * kHD + d;
    if constexpr (HAS2) n2 = (effective_len(a.r2, b, a.log2_bs) + chunk_len - 1) / chunk_len;
    const int n4 = (effective_len(a.r4, b, a.log2_bs) + chunk_len - 1) / chunk_len;
    const int n8 = (effective_len(a.r8, b, a.log2_bs) + chunk_len - 1) / chunk_len;
    if constexpr (LIVE) cend = min(cend, n8);      // one int8 region: chunks [0, n8) are live
    float M = -INFINITY, S = 0.0f, acc = 0.0f;
    for (int c0 = cbeg; c0 < cend; c0 += BATCH) {
        float mv[BATCH], sv[BATCH], av[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int cc = min(c0 + k, cend - 1);
            // M and S are the same for every thread of the part; as scalar
            // loads they ran out of scalar registers and were waited for in
            // turn.  Vector loads of the same word go out with the acc loads.
            int cv = cc;
            __asm__("" : "+v"(cv));
            mv[k] = mm[cv];
            sv[k] = ss[cv];
            av[k] = aa[(size_t)cc * kHD];
        }
        float bm = -INFINITY;
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int c = c0 + k;
            bool live;
            if constexpr (HAS2)
                live = c < cend && (c < n2 || (c >= base4 && c < base4 + n4) || (c >= base8 && c < base8 + n8));
            else
                live = c < cend && (c < n4 || (c >= base8 && c < base8 + n8));
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
        for (int k = 0; k < BATCH; ++k) {
            const float f = __builtin_amdgcn_exp2f(mv[k] - M);
            S = fmaf(sv[k], f, S);
            acc = fmaf(av[k], f, acc);
        }
    }
    if (part > 0) {
        other[part][d] = acc;
        if (d == 0) {
            other[part][kHD] = M;
            other[part][kHD + 1] = S;
        }
    }
    __syncthreads();
    if (part == 0) {
        float Mt = M;
#pragma unroll
        for (int q = 1; q < PARTS; ++q) Mt = fmaxf(Mt, other[q][kHD]);
        float res = 0.0f;
        if (Mt != -INFINITY) {
            const float f0 = __builtin_amdgcn_exp2f(M - Mt);
            float num = acc * f0, den = S * f0;
#pragma unroll
            for (int q = 1; q < PARTS; ++q) {
                const float f = __builtin_amdgcn_exp2f(other[q][kHD] - Mt);
                num = fmaf(other[q][d], f, num);
                den = fmaf(other[q][kHD + 1], f, den);
            }
            res = num / den;
        }
        out[(size_t)bh * kHD + d] = res;
    }
}

// The merge of one region for a single sequence (a batch-1 int8 or Q4_0
// decode, where the merge is on the step's critical path): the arguments in
// one batch, and the length read after the partials' loads are issued, so
// that one memory round trip serves them all.
template <int PARTS>
__global__ __launch_bounds__(PARTS * kHD) void kvq_merge1_kernel(float* __restrict__ out, DecodeArgs a) {
    __shared__ float other[PARTS][kHD + 2];
    {
        const void* p0 = a.ws_acc;
        const void* p1 = a.ws_m;
        const void* p2 = a.ws_s;
        const void* p3 = a.r8.lens;
        const void* p4 = out;
        __asm__ volatile("" ::"s"(p0), "s"(p1), "s"(p2), "s"(p3), "s"(p4), "s"(a.nq), "s"(a.tiles_per_wave),
                         "s"(a.r8.max_chunks), "s"(a.r8.max_len), "s"(a.r8.max_blocks), "s"(a.log2_bs));
    }
    const int bh = blockIdx.x;
    const int b = bh / a.nq;
    const int d = threadIdx.x & (kHD - 1);
    const int part = __builtin_amdgcn_readfirstlane(threadIdx.x / kHD);
    const int chunk_len = a.tiles_per_wave * kChunkUnit;
    const int nct = a.r8.max_chunks;
    const int share = (nct + PARTS - 1) / PARTS;
    const int cbeg = part * share;
    const int cend = min(nct, cbeg + share);
    const float* mm = a.ws_m + (size_t)bh * nct;
    const float* ss = a.ws_s + (size_t)bh * nct;
    const float* aa = a.ws_acc + (size_t)bh * nct * kHD + d;
    // the length bound: max_len, and what the block table can hold
    const int lim = (int)min((long)a.r8.max_len, (long)a.r8.max_blocks << a.log2_bs);
    float M = -INFINITY, S = 0.0f, acc = 0.0f;
    for (int c0 = cbeg; c0 < cend; c0 += kMergeBatch) {
        float mv[kMergeBatch], sv[kMergeBatch], av[kMergeBatch];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            int cv = min(c0 + k, cend - 1);
            __asm__("" : "+v"(cv));
            mv[k] = mm[cv];
            sv[k] = ss[cv];
            av[k] = aa[(size_t)cv * kHD];
        }
        int bv = b;
        __asm__("" : "+v"(bv));
        const int lraw = a.r8.lens[bv];
        // every load of the batch is issued before anything waits on one
        __builtin_amdgcn_sched_barrier(0);
        const int L = min(lraw, lim);
        const int n8 = L > 0 ? (int)((unsigned)(L + chunk_len - 1) / (unsigned)chunk_len) : 0;
        float bm = -INFINITY;
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const int c = c0 + k;
            const bool live = c < cend && c < n8;
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
    if (part > 0) {
        other[part][d] = acc;
        if (d == 0) {
            other[part][kHD] = M;
            other[part][kHD + 1] = S;
        }
    }
    __syncthreads();
    if (part == 0) {
        float Mt = M;
#pragma unroll
        for (int q = 1; q < PARTS; ++q) Mt = fmaxf(Mt, other[q][kHD]);
        float res = 0.0f;
        if (Mt != -INFINITY) {
            const float f0 = __builtin_amdgcn_exp2f(M - Mt);
            float num = acc * f0, den = S * f0;
#pragma unroll
            for (int q = 1; q < PARTS; ++q) {
                const float f = __builtin_amdgcn_exp2f(other[q][kHD] - Mt);
                num = fmaf(other[q][d], f, num);
                den = fmaf(other[q][kHD + 1], f, den);
            }
            res = num / den;
        }
        out[(size_t)bh * kHD + d] = res;
    }
}

// Enqueue the merge of a decode's chunk partials into `out`.
// A part's share of at most kMergeBatch / 2 chunks is read in one half-size
// batch (the other half of a full batch would only repeat its last chunk).
inline bool half_batch(int n_chunks, int parts) { return (n_chunks + parts - 1) / parts <= kMergeBatch / 2; }

inline int launch_merge(const BandArgs& a, float* out, hipStream_t s) {
    const dim3 grid(a.batch * a.nq);
    constexpr int H = kMergeBatch / 2;
    const int nct = n_chunks_total(a);
    if (nct > 2 * kMergeBatch)
        return half_batch(nct, 8)
                   ? launch((kvq_merge_kernel<8, false, BandArgs, H>), grid, dim3(kMergeThreadsWide), s, out, a)
                   : launch((kvq_merge_kernel<8, false, BandArgs>), grid, dim3(kMergeThreadsWide), s, out, a);
    return half_batch(nct, 2) ? launch((kvq_merge_kernel<2, false, BandArgs, H>), grid, dim3(kMergeThreads), s, out, a)
                              : launch((kvq_merge_kernel<2, false, BandArgs>), grid, dim3(kMergeThreads), s, out, a);
}

inline int launch_merge(const DecodeArgs& a, float* out, hipStream_t s) {
    const bool live = a.batch > 1 && a.r4.max_chunks == 0;
    const bool wide = n_chunks_total(a) > 2 * kMergeBatch;
    const dim3 grid(a.batch * a.nq), block(wide ? kMergeThreadsWide : kMergeThreads);
    if (a.batch == 1 && a.r4.max_chunks == 0)
        return wide ? launch((kvq_merge1_kernel<8>), grid, block, s, out, a)
                    : launch((kvq_merge1_kernel<2>), grid, block, s, out, a);
    constexpr int H = kMergeBatch / 2;
    const int nct = n_chunks_total(a);
    if (wide) {
        if (half_batch(nct, 8))
            return live ? launch((kvq_merge_kernel<8, true, DecodeArgs, H>), grid, block, s, out, a)
                        : launch((kvq_merge_kernel<8, false, DecodeArgs, H>), grid, block, s, out, a);
        return live ? launch((kvq_merge_kernel<8, true>), grid, block, s, out, a)
                    : launch((kvq_merge_kernel<8, false>), grid, block, s, out, a);
    }
    if (half_batch(nct, 2))
        return live ? launch((kvq_merge_kernel<2, true, DecodeArgs, H>), grid, block, s, out, a)
                    : launch((kvq_merge_kernel<2, false, DecodeArgs, H>), grid, block, s, out, a);
    return live ? launch((kvq_merge_kernel<2, true>), grid, block, s, out, a)
                : launch((kvq_merge_kernel<2, false>), grid, block, s, out, a);
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

// Tokens per chunk: the largest power-of-two multiple of 256 that still gives
// at least `min_wg` workgroups (default one per CU), capped at `max_tpw` x 256
// tokens.  `units` = sequences x kv-heads, `max_len` the longest region.
inline int default_tiles_per_wave(long units, long max_len, int max_tpw, long min_wg = 256) {
    int tpw = 1;
    while (tpw < max_tpw) {
        const long next = (long)kChunkUnit * tpw * 2;
        if (units * ((max_len + next - 1) / next) < min_wg) break;
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

// The partials' places in the workspace (every region set first).
template <class Args>
inline void bind_workspace(Args& a, void* workspace) {
    const size_t n = (size_t)a.batch * a.nq * n_chunks_total(a);
    char* ws = static_cast<char*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(ws);
    a.ws_m = reinterpret_cast<float*>(ws + round_up(n * kHD * sizeof(float), 256));
    a.ws_s = reinterpret_cast<float*>(ws + round_up(n * kHD * sizeof(float), 256) + round_up(n * sizeof(float), 256));
}

}  // namespace kvq
