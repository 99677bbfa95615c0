// sp_host_checks.h -- host-side argument checks shared by the C entry
// points: pointer ranges, overlap and alignment.
#pragma once

#include <stdint.h>

namespace spr {

struct Range {
    uintptr_t lo, hi;   // [lo, hi); empty when lo == hi
};

inline Range range_of(const void* p, uint64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return p ? Range{a, a + (uintptr_t)bytes} : Range{0, 0};
}

inline bool overlaps(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

inline bool aligned(const void* p, uintptr_t n) {
    return (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

// Outputs must not overlap each other or any input.
inline bool disjoint(const Range* outs, int nout, const Range* ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i], outs[j])) return false;
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i], ins[j])) return false;
    }
    return true;
}

}  // namespace spr
