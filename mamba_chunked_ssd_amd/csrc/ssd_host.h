// ssd_host.h -- host helpers shared by the C-ABI translation units
// (ssd_api.cpp, ssd_bwd.cpp): shape validation and pointer checks.  Host code
// only.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/ssd.h"
#include "ssd_internal.h"

namespace ssd {

constexpr size_t kAlign = 256;  // workspace alignment and region granularity

size_t align_up(size_t v);

// The checks every entry point applies to a shape and chunk size; fills *p.
ssd_status check_shape(const ssd_shape *s, int64_t chunk, Problem *p);

inline bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
inline Range range_of(const void *ptr, size_t bytes) { return Range{(uintptr_t)ptr, (uintptr_t)ptr + bytes}; }
inline bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

}  // namespace ssd
