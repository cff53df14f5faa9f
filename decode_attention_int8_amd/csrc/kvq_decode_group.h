// The group-variant decode kernel: chunks of the 2-bit band, of the int4
// band and of the int8 window share one launch and one merge ([P4] Sec. 3.3
// bands over the [P3] Sec. 2 single pass); int8 chunks run the int8 tile
// code, the two group bands one walk over their own tiles.
#pragma once

#include "kvq_decode_mfma2.h"

namespace kvq {

// The tile operations of the two group formats, for the shared walk.
template <class Tile>
struct GroupTileOps;

template <>
struct GroupTileOps<MTile4> {
    using Off = LaneOff4;
    static constexpr bool kEvenOdd = true;        // query operand order of the int4 key unpacking
    static __device__ __forceinline__ Off offsets(const DecodeArgs& a, int lane) { return lane_offsets4(a, lane); }
    template <bool BS8>
    static __device__ __forceinline__ void issue(const DecodeArgs& a, int raw, int base, int kh, int lane,
                                                 const Off& lo, MTile4& T) {
        mtile4_issue<BS8>(a, raw, base, kh, lane, lo, T);
    }
    static __device__ __forceinline__ void compute(const DecodeArgs& a, const MTile4& T, int base, int L, int lane,
                                                   int wave, const MQuery4& Q, MStateG& st, MSmem4& sm) {
        mtile4_compute(a, T, base, L, lane, wave, Q, st, sm);
    }
};

template <>
struct GroupTileOps<MTile2> {
    using Off = LaneOff2;
    static constexpr bool kEvenOdd = false;
    static __device__ __forceinline__ Off offsets(const BandArgs& a, int lane) { return lane_offsets2(a, lane); }
    template <bool BS8>
    static __device__ __forceinline__ void issue(const BandArgs& a, int raw, int base, int kh, int lane,
                                                 const Off& lo, MTile2& T) {
        mtile2_issue<BS8>(a, raw, base, kh, lane, lo, T);
    }
    static __device__ __forceinline__ void compute(const BandArgs& a, const MTile2& T, int base, int L, int lane,
                                                   int wave, const MQuery4& Q, MStateG& st, MSmem4& sm) {
        mtile2_compute(a, T, base, L, lane, wave, Q, st, sm);
    }
};

// One workgroup's walk over a chunk of a group band: double-buffered tiles,
// two per trip with one exit test at the top; the table entries of the tile
// after next go out before a tile's loads, so the loop head waits for them
// without waiting for the tile.
template <bool BS8, class Tile, class Args>
__device__ __forceinline__ void group_walk(const Args& a, const Region& reg, const int32_t* btb, int raw,
                                           int first, int L, int n_tiles, const float4& qx, int G, int b, int kh,
                                           int c, int lane, int wave, MSmem4& sm) {
    using Ops = GroupTileOps<Tile>;
    const int g = lane >> 4;
    const int m = lane & 15;
    const typename Ops::Off lo = Ops::offsets(a, lane);
    Tile A, B;
    int raw_next = mtile_raw(reg, btb, first + kChunkUnit, a.log2_bs, lane);
    Ops::template issue<BS8>(a, raw, first, kh, lane, lo, A);
    raw = raw_next;
    __asm__ volatile("" ::: "memory");
    quantize_q4(qx, G, sm.q);
    lds_barrier();
    const MQuery4 Q = load_q4_operand<Ops::kEvenOdd>(sm.q, G, g, m);
    MStateG st;
    st.M = -INFINITY;
    st.S = 0.0f;
    st.E = 100;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) st.acc[sl] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
    st.accz[0] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
    st.accz[1] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
    int base = first;
    int k = 0;
    for (; k + 2 < n_tiles; k += 2) {
        raw_next = mtile_raw(reg, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
        Ops::template issue<BS8>(a, raw, base + kChunkUnit, kh, lane, lo, B);
        raw = raw_next;
        // the tile's vector work ahead of the other wave's loads on this SIMD
        // (int4 128K decode ~3% faster; the 2-bit band unchanged)
        __builtin_amdgcn_s_setprio(2);
        Ops::compute(a, A, base, L, lane, wave, Q, st, sm);
        __builtin_amdgcn_s_setprio(0);
        base += kChunkUnit;
        raw_next = mtile_raw(reg, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
        Ops::template issue<BS8>(a, raw, base + kChunkUnit, kh, lane, lo, A);
        raw = raw_next;
        __builtin_amdgcn_s_setprio(2);
        Ops::compute(a, B, base, L, lane, wave, Q, st, sm);
        __builtin_amdgcn_s_setprio(0);
        base += kChunkUnit;
    }
    if (k + 1 < n_tiles) {
        Ops::template issue<BS8>(a, raw, base + kChunkUnit, kh, lane, lo, B);
        Ops::compute(a, A, base, L, lane, wave, Q, st, sm);
        Ops::compute(a, B, base + kChunkUnit, L, lane, wave, Q, st, sm);
    } else {
        Ops::compute(a, A, base, L, lane, wave, Q, st, sm);
    }
    mwave4_to_lds(sm, st, G, lane, wave);
    lds_barrier();
    mcombine_write(a, sm, G, b, kh, c);
}

// One workgroup = (sequence, kv-head, chunk) of any band: chunks
// [0, r2.max_chunks) cover the 2-bit band (BandArgs only), the next
// r4.max_chunks the int4 band, the rest the int8 window.  Two workgroups per
// CU (the int8 walk issues values after P.V, as in the int8 kernel).
template <bool BS8, class Args>
__global__ __launch_bounds__(kWGThreads, 2) void kvq4_decode_mfma_kernel(Args a) {
    constexpr bool HAS2 = kBanded<Args>;
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
    // The heaviest chunks first: rank r = p / batch runs over the int8
    // window's chunks, then the int4 band's, then the 2-bit band's, each for
    // every sequence (b = p % batch), so the workgroups dispatched last are the
    // lightest ones.  Pair p runs on XCD p % 8 with its nkv workgroups.
    int m2 = 0;
    if constexpr (HAS2) m2 = a.r2.max_chunks;
    const int n4c = a.r4.max_chunks, n8c = a.r8.max_chunks;
    const int b = p % a.batch;
    const int r = p / a.batch;
    if (r >= nct) return;
    const int c = r < n8c ? m2 + n4c + r : (r < n8c + n4c ? m2 + (r - n8c) : r - n8c - n4c);
    const int kind = (HAS2 && c < m2) ? 2 : (c < m2 + a.r4.max_chunks ? 4 : 8);
    const Region* regp = kind == 4 ? &a.r4 : &a.r8;
    if constexpr (HAS2) {
        if (kind == 2) regp = &a.r2;
    }
    const Region& reg = *regp;
    const int cr = (HAS2 && kind == 2) ? c : (kind == 4 ? c - m2 : c - m2 - a.r4.max_chunks);
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

    if (kind == 4) {
        group_walk<BS8, MTile4>(a, reg, btb, raw, first, L, n_tiles, qx, G, b, kh, c, lane, wave, sm);
    } else if (kind == 2) {
        if constexpr (HAS2)
            group_walk<BS8, MTile2>(a, reg, btb, raw, first, L, n_tiles, qx, G, b, kh, c, lane, wave, sm);
    } else {
        const LaneOff lo = lane_offsets(a, lane, kh);
        MTile A, B;
        mtile_issue<BS8, kIssueKeys | kIssueSteps>(a, raw, first, kh, lane, lo, A);
        raw = mtile_raw(reg, btb, first + kChunkUnit, a.log2_bs, lane);
        mtile_issue<BS8, kIssueValues>(a, 0, first, kh, lane, lo, A);
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
        int k = 0;
        for (; k + 2 < n_tiles; k += 2) {
            mtile_issue<BS8, kIssueKeys | kIssueSteps>(a, raw, base + kChunkUnit, kh, lane, lo, B);
            raw = mtile_raw(reg, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
            mtile_compute(a, A, base, L, lane, wave, Q, st, sm, NoHook(), [&]() __attribute__((always_inline)) {
                mtile_issue<BS8, kIssueValues>(a, 0, base + kChunkUnit, kh, lane, lo, B);
            });
            base += kChunkUnit;
            mtile_issue<BS8, kIssueKeys | kIssueSteps>(a, raw, base + kChunkUnit, kh, lane, lo, A);
            raw = mtile_raw(reg, btb, base + 2 * kChunkUnit, a.log2_bs, lane);
            mtile_compute(a, B, base, L, lane, wave, Q, st, sm, NoHook(), [&]() __attribute__((always_inline)) {
                mtile_issue<BS8, kIssueValues>(a, 0, base + kChunkUnit, kh, lane, lo, A);
            });
            base += kChunkUnit;
        }
        if (k + 1 < n_tiles) {
            mtile_issue<BS8, kIssueKeys | kIssueSteps>(a, raw, base + kChunkUnit, kh, lane, lo, B);
            mtile_compute(a, A, base, L, lane, wave, Q, st, sm, NoHook(), [&]() __attribute__((always_inline)) {
                mtile_issue<BS8, kIssueValues>(a, 0, base + kChunkUnit, kh, lane, lo, B);
            });
            mtile_compute(a, B, base + kChunkUnit, L, lane, wave, Q, st, sm);
        } else {
            mtile_compute(a, A, base, L, lane, wave, Q, st, sm);
        }
        mwrite_partial(a, sm, st, G, b, kh, c, lane, wave);
    }
}

template <class Args>
inline int launch_mfma4(const Args& a, int n_wg, hipStream_t s) {
    const dim3 grid(n_wg), block(kWGThreads);
    if (a.log2_bs < 4) return launch((kvq4_decode_mfma_kernel<true, Args>), grid, block, s, a);
    return launch((kvq4_decode_mfma_kernel<false, Args>), grid, block, s, a);
}

// Enqueue the chunk kernel (if there is any context) and the merge kernel.
// new_dtype >= 0 fuses the write path of each sequence's last token.  The
// int8 cache and the banded group caches all run on the matrix cores.
template <class Args>
inline int launch_decode(const Args& a, float* out, hipStream_t s, int new_dtype = -1) {
    const int nct = n_chunks_total(a);
    if (nct > 0) {
        const long pairs = (long)a.batch * pair_stride(nct, a.batch);
        const long n_wg = (long)a.nkv * ((pairs + 7) / 8) * 8;
        if (n_wg > 0x7FFFFFFFL) return KVQ8_ESHAPE;
        int st;
        if constexpr (kBanded<Args>)
            st = launch_mfma4(a, (int)n_wg, s);
        else if (a.r4.max_chunks > 0)
            st = launch_mfma4(a, (int)n_wg, s);
        else
            st = launch_mfma(a, (int)n_wg, new_dtype, s);
        if (st != KVQ8_OK) return st;
    }
    return launch_merge(a, out, s);
}

}  // namespace kvq
