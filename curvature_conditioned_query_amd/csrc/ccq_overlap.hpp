// Byte-range overlap of a prefill's carry out with its carry in (host code only, no HIP).
//
// With more than one segment per chain, segment 0 of the main kernel reads the caller's carry in
// while the chain's last segment writes the carry out in the same launch, in no fixed order.  When
// the two overlap, the library copies the carry in to the workspace first; this decides when.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ccq {

struct CarryRanges {
  const void *S, *C, *ksum, *n;  // all four set, or S == nullptr (absent)
};

// Whether any byte of `out` lies in `in`, for `chains` (b, h) chains of head dimension d; C holds
// d (d + 1) / 2 floats per chain when packed, else d * d.
inline bool carry_ranges_overlap(const CarryRanges& in, const CarryRanges& out, size_t chains, size_t d,
                                 bool packed) {
  if (in.S == nullptr || out.S == nullptr) return false;
  const size_t cn = packed ? d * (d + 1) / 2 : d * d;
  const size_t bytes[4] = {chains * d * d * 4, chains * cn * 4, chains * d * 4, chains * 8};
  const void* a[4] = {in.S, in.C, in.ksum, in.n};
  const void* b[4] = {out.S, out.C, out.ksum, out.n};
  for (int i = 0; i < 4; ++i) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(a[i]), hi = lo + bytes[i];
    for (int j = 0; j < 4; ++j) {
      const uintptr_t lo2 = reinterpret_cast<uintptr_t>(b[j]), hi2 = lo2 + bytes[j];
      if (lo < hi2 && lo2 < hi) return true;
    }
  }
  return false;
}

}  // namespace ccq
