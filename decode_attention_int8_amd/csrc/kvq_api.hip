// Status strings and version of the library.
#include "kvq8.h"

extern "C" const char* kvq8_status_string(int status) {
    switch (status) {
        case KVQ8_OK: return "ok";
        case KVQ8_EINVAL: return "invalid argument (null pointer, misalignment, negative count or unknown dtype)";
        case KVQ8_ESHAPE: return "unsupported shape (hd, kv_bs, head grouping, chunk or grid size)";
        case KVQ8_EWORKSPACE: return "workspace missing, misaligned or too small";
        case KVQ8_EHIP: return "HIP launch or runtime error";
        default: return "unknown status";
    }
}

extern "C" const char* kvq8_version(void) { return "kvq8 1.0 gfx950"; }
