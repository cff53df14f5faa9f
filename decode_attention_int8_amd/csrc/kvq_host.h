// Host-side helpers shared by the entry points: argument checks and launch
// status.  No device code and no allocation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <cmath>
#include <tuple>

#include "kvq8.h"

namespace kvq {

inline bool valid_block_size(int kv_bs) {
    return kv_bs >= 8 && kv_bs <= 1024 && (kv_bs & (kv_bs - 1)) == 0;
}

inline int ilog2(int v) {
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Enqueue `kernel` on stream `s` with `args` (converted to the kernel's
// parameter types) and return the status of this launch alone: KVQ8_EHIP if
// hipLaunchKernel rejects it, else KVQ8_OK.  The runtime's pending error
// state is neither read nor cleared, so an error left by an earlier, unrelated
// call is not reported here and stays for its owner to collect.
template <typename... P, typename... A>
inline int launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, A... args) {
    static_assert(sizeof...(P) == sizeof...(A), "argument count differs from the kernel's");
    std::tuple<P...> vals(args...);
    void* ptrs[sizeof...(P)];
    std::apply([&ptrs](auto&... v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
    }, vals);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, s) == hipSuccess
               ? KVQ8_OK
               : KVQ8_EHIP;
}

// The score scale of the decodes: sm_scale when positive; 0 or a negative
// value selects the method's 1 / sqrt(hd) with hd = 128 ([P1] "Day 9-3"
// Sec. 1-2: scores are divided by the square root of 128).  A NaN or
// infinite value is an invalid argument.
inline bool score_scale_ok(float sm_scale) { return std::isfinite(sm_scale); }

inline float score_scale(float sm_scale) { return sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf(128.0f); }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The slot bound a write kernel tests with one unsigned compare: min(n_slots,
// 2^31), so that (uint32_t)slot < slot_cap(n_slots) holds exactly for an
// int32 slot in [0, n_slots).
inline uint32_t slot_cap(long n_slots) { return (uint32_t)(n_slots < 0x80000000L ? n_slots : 0x80000000L); }

}  // namespace kvq
