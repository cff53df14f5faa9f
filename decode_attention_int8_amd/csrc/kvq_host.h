// Host-side helpers shared by the entry points: argument checks and launch
// status.  No device code and no allocation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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

// Status of the launches just enqueued: KVQ8_EHIP if the runtime reports an
// error, else KVQ8_OK.
inline int launch_status() {
    return hipGetLastError() == hipSuccess ? KVQ8_OK : KVQ8_EHIP;
}

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace kvq
