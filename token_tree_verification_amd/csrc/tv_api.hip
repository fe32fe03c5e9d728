// Status strings and version of the libtv C ABI.
#include "tv_internal.h"

extern "C" const char* tv_status_string(int status) {
    switch (status) {
        case TV_OK: return "ok";
        case TV_ERR_INVALID_ARG: return "invalid argument";
        case TV_ERR_UNSUPPORTED: return "unsupported shape (N > 256 or head dim != 128)";
        case TV_ERR_BAD_TREE: return "invalid tree: parent[0] must be -1 and 0 <= parent[i] < i";
        case TV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case TV_ERR_HIP: return "HIP launch or runtime error";
        case TV_ERR_SCRATCH: return "shape needs more scratch than the allocation-free call holds";
        default: return "unknown status";
    }
}

extern "C" int tv_version(void) { return 100; }
