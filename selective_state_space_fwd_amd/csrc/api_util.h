// Argument-checking helpers shared by the C-ABI entry points (host only).
#pragma once
#include <stdint.h>

namespace ssm_api {

constexpr int64_t kInt32Max = 2147483647;

// a * b with overflow detection for non-negative operands.
inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

inline bool overlaps(Range x, Range y) { return x.lo < y.hi && y.lo < x.hi; }

inline Range span(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace ssm_api
