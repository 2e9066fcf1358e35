// Shared host/device helpers of libgraft (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "graft.h"

namespace graft {

// Records a printf-style message for graft_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Returns GRAFT_OK, or GRAFT_EHIP with the HIP error text if the last launch failed.
int check_launch(const char *what);
void clear_error();

inline hipStream_t as_stream(graft_stream s) { return reinterpret_cast<hipStream_t>(s); }
// Arrays the kernels read or write 16 bytes at a time must start on a
// 16-byte boundary (every PyTorch allocation does).
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ORs error bits into the caller's device flag word (vector-memory atomic).
__device__ inline void raise_flag(int32_t *err, int bits) {
  if (err) atomicOr(err, bits);
}

// (value, id) ordering used by every ranking: larger value first, ties to
// the lower id.  NaN never ranks above anything.
__device__ inline bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Order-preserving 32-bit image of a float (larger float -> larger integer);
// -0 is first folded into +0 so that the two compare equal.  Every NaN maps
// to 0, below -inf (0x007FFFFF), so a NaN ranks after every number and NaNs
// tie with each other (ties go to the lower id).
__device__ inline uint32_t float_order(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return x == x ? o : 0u;
}

}  // namespace graft
