// The int8 decode chunk kernel on the matrix cores and its launchers (the
// tile machinery is in kvq_decode_mfma.h).
#pragma once

#include "kvq_decode_mfma.h"

namespace kvq {

// Two workgroups per CU: the walk fits the 256 registers of that budget
// because a tile's values are issued only after the previous tile's P.V,
// when its values are dead (one value buffer, two key buffers).
template <int NEWDT, bool BS8, bool DENSE>
__global__ __launch_bounds__(kWGThreads, 2) void kvq_decode_mfma_kernel(DecodeArgs a) {
    __shared__ MSmem sm;
    // The arguments the prologue needs, read in one batch: left to itself
    // the compiler loads each at its first use, behind the previous wait, and
    // at batch 1 (every workgroup its CU's first) those round trips add up.
    {
        const void* p0 = a.q;
        const void* p1 = a.r8.bt;
        const void* p2 = a.r8.lens;
        const void* p3 = a.kc;
        const void* p4 = a.ks;
        __asm__ volatile("" ::"s"(p0), "s"(p1), "s"(p2), "s"(p3), "s"(p4), "s"(a.nq), "s"(a.nkv), "s"(a.batch),
                         "s"(a.r8.max_chunks), "s"(a.tiles_per_wave), "s"(a.r8.max_blocks), "s"(a.r8.max_len),
                         "s"(a.log2_bs), "s"(a.r8.n_blocks));
        if constexpr (NEWDT >= 0) {
            const void* p5 = a.k_new;
            const void* p6 = a.v_new;
            __asm__ volatile("" ::"s"(p5), "s"(p6));
        }
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = a.nq / a.nkv;

    // work decode: the nkv workgroups of one (sequence, chunk) pair share an
    // XCD (pair p on XCD p % 8).  Batches take the dense pair order of
    // dense_item; otherwise pairs are laid out at an odd stride.
    const int nct = a.r8.max_chunks;
    const int wg = blockIdx.x;
    const int rest = wg >> 3;
    const int kh = rest % a.nkv;
    const int p = (rest / a.nkv) * 8 + (wg & 7);
    const int chunk_len = a.tiles_per_wave * kChunkUnit;
    int b, c, raw, L, lraw;     // lraw: the length as given (read once, for the fused write path)
    float4 qx;
    if constexpr (DENSE) {
        DenseItem it;
        if (!dense_item(a.r8, a.batch, a.log2_bs, chunk_len, p, lane, it)) return;
        b = it.b;
        c = it.c;
        L = it.L;
        lraw = it.lraw;
        raw = mtile_raw(a.r8, a.r8.bt + (size_t)b * a.r8.max_blocks, c * chunk_len + wave * kTile, a.log2_bs, lane);
        qx = load_q4(a.q + ((size_t)b * a.nq + (size_t)kh * G) * kHD, G);
    } else {
        b = p / pair_stride(nct, a.batch);
        c = p - b * pair_stride(nct, a.batch);
        if (b >= a.batch || c >= nct) return;
        raw = mtile_raw(a.r8, a.r8.bt + (size_t)b * a.r8.max_blocks, c * chunk_len + wave * kTile, a.log2_bs, lane);
        // the query rows do not depend on the length: their loads go out with
        // the table entries, so their quantization never waits on the tile
        qx = load_q4(a.q + ((size_t)b * a.nq + (size_t)kh * G) * kHD, G);
        L = effective_len(a.r8, b, a.log2_bs, lraw);
        if (c * chunk_len >= L) return;                        // uniform per workgroup
    }
    const int c0 = c * chunk_len;
    const int32_t* btb = a.r8.bt + (size_t)b * a.r8.max_blocks;
    const int first = c0 + wave * kTile;
    const int end = min(L, c0 + chunk_len);
    // tiles of this wave: first, first + 256, ... (at least one, possibly empty)
    const int n_tiles = first < end ? (end - first + kChunkUnit - 1) / kChunkUnit : 1;

    // fused write path: one wave owns the token at L-1.  A length above the
    // bound (clamped to L) puts the new token past what the call attends:
    // it is then neither written nor attended, and tn = -1 matches no token.
    const int tn = lraw == L ? L - 1 : -1;
    const bool has_new = NEWDT >= 0 && tn >= c0 && tn < end && (((tn - c0) >> 6) & (kWaves - 1)) == wave;
    // then the new token's loads, then the first tile's.  Every wave loads
    // the new rows (L2 hits after the first): a load in a branch leaves the
    // compiler's wait before the tile's loads counting it, so that the owner
    // wave would wait a round trip before issuing its tile.
    float xn[4];
    if constexpr (NEWDT >= 0) {
        // lanes 0-31: K row, lanes 32-63: V row, 4 values each
        load_new4<NEWDT>(lane < 32 ? a.k_new : a.v_new, ((size_t)b * a.nkv + kh) * kHD + 4 * (lane & 31), xn);
    }

    const LaneOff lo = lane_offsets(a, lane, kh);
    MTile A, B;
    // the same issue order as the walk (keys and steps, the next table entries,
    // values), so that the loop head's wait for those entries is the same
    // count on entry as on the back edge instead of a wait for everything
    mtile_issue<BS8, kIssueKeys | kIssueSteps>(a, raw, first, kh, lane, lo, A);
    raw = mtile_raw(a.r8, btb, first + kChunkUnit, a.log2_bs, lane);
    mtile_issue<BS8, kIssueValues>(a, 0, first, kh, lane, lo, A);
    __asm__ volatile("" ::: "memory");

    quantize_q4(qx, G, sm.q);
    if constexpr (NEWDT >= 0) {
        if (has_new) {
            // the new token's codes and steps go to LDS; its terminal tile
            // takes them in place of the slot's stale copy and stores them
            uint32_t codes;
            float d;
            quantize_row32x4(xn, codes, d);
            reinterpret_cast<uint32_t*>(lane < 32 ? sm.nk : sm.nv)[lane & 31] = codes;
            if ((lane & 31) == 0) sm.nstep[lane >> 5] = d;
        }
    }
    lds_barrier();
    const int g = lane >> 4;
    const int m = lane & 15;
    const MQuery Q = load_q_operand(sm.q, G, g, m);

    MState st;
    st.M = -INFINITY;
    st.S = 0.0f;
    st.E = 100;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) st.acc[sl] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Token tn = L-1 is the last token of the sequence, so it can only lie in
    // the last tile of a wave: only the two terminal calls substitute, with
    // selects that match nothing outside the owner's tile (and nothing at all
    // when tn = -1).
    auto run_last = [&](const MTile& T, int base) __attribute__((always_inline)) {
        if constexpr (NEWDT >= 0) {
            if (has_new) {
                // store the new token into its cache slot: the block id is the
                // tile's own table entry of position tn (-1 outside the pool)
                const int bid = __builtin_amdgcn_readlane(T.id, tn - base);
                if (bid >= 0) {
                    const size_t slot = ((size_t)bid << a.log2_bs) + (tn & ((1 << a.log2_bs) - 1));
                    const size_t row = slot * a.nkv + kh;
                    const size_t crow = slot * a.nkv + q8_col(kh, (long)slot, q8_rot_group(a.nkv));
                    const uint32_t w = reinterpret_cast<const uint32_t*>(lane < 32 ? sm.nk : sm.nv)[lane & 31];
                    *reinterpret_cast<uint32_t*>((lane < 32 ? a.kc_w : a.vc_w) + crow * kHD + 4 * (lane & 31)) = w;
                    if ((lane & 31) == 0) (lane < 32 ? a.ks_w : a.vs_w)[row] = sm.nstep[lane >> 5];
                }
            }
            mtile_compute(a, mtile_substitute(T, sm, base, tn, lane), base, L, lane, wave, Q, st, sm);
        } else {
            mtile_compute(a, T, base, L, lane, wave, Q, st, sm);
        }
    };
    // double-buffered walk: tile k+1's keys and steps are in flight while
    // tile k is computed, its values from the end of tile k's P.V on; the
    // table entries run one tile further ahead
    int base = first;
    for (int k = 0;;) {
        if (k + 1 >= n_tiles) {
            run_last(A, base);
            break;
        }
        mtile_issue<BS8, kIssueKeys | kIssueSteps>(a, raw, base + kChunkUnit, kh, lane, lo, B);
        raw = mtile_raw(a.r8, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
        mtile_compute(a, A, base, L, lane, wave, Q, st, sm, NoHook(), [&]() __attribute__((always_inline)) {
            mtile_issue<BS8, kIssueValues>(a, 0, base + kChunkUnit, kh, lane, lo, B);
        });
        base += kChunkUnit;
        ++k;
        if (k + 1 >= n_tiles) {
            run_last(B, base);
            break;
        }
        mtile_issue<BS8, kIssueKeys | kIssueSteps>(a, raw, base + kChunkUnit, kh, lane, lo, A);
        raw = mtile_raw(a.r8, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
        mtile_compute(a, B, base, L, lane, wave, Q, st, sm, NoHook(), [&]() __attribute__((always_inline)) {
            mtile_issue<BS8, kIssueValues>(a, 0, base + kChunkUnit, kh, lane, lo, A);
        });
        base += kChunkUnit;
        ++k;
    }
    mwrite_partial(a, sm, st, G, b, kh, c, lane, wave);
}

template <bool BS8, bool DENSE>
inline int launch_mfma_bs(const DecodeArgs& a, int n_wg, int new_dtype, hipStream_t s) {
    const dim3 grid(n_wg), block(kWGThreads);
    if (new_dtype == KVQ8_F32) return launch((kvq_decode_mfma_kernel<KVQ8_F32, BS8, DENSE>), grid, block, s, a);
    if (new_dtype == KVQ8_BF16) return launch((kvq_decode_mfma_kernel<KVQ8_BF16, BS8, DENSE>), grid, block, s, a);
    if (new_dtype == KVQ8_F16) return launch((kvq_decode_mfma_kernel<KVQ8_F16, BS8, DENSE>), grid, block, s, a);
    return launch((kvq_decode_mfma_kernel<-1, BS8, DENSE>), grid, block, s, a);
}

// Batches of 2 .. 64 sequences take the dense work order (one more memory
// round trip per workgroup, for the lengths, before its table entries; a
// single sequence has nothing to balance and keeps that round trip off its
// critical path).
inline int launch_mfma(const DecodeArgs& a, int n_wg, int new_dtype, hipStream_t s) {
    const bool dense = a.batch > 1 && a.batch <= kDenseMaxBatch;
    if (a.log2_bs < 4)
        return dense ? launch_mfma_bs<true, true>(a, n_wg, new_dtype, s) : launch_mfma_bs<true, false>(a, n_wg, new_dtype, s);
    return dense ? launch_mfma_bs<false, true>(a, n_wg, new_dtype, s) : launch_mfma_bs<false, false>(a, n_wg, new_dtype, s);
}

}  // namespace kvq
