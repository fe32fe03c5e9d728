// Host-side declarations shared by the libtv translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tv.h"

namespace tv {

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int launch_status() { return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP; }

}  // namespace tv
