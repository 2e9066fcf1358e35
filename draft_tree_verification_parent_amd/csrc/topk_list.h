// Per-thread sorted top-K lists over (value desc, id asc), as 64-bit keys.
//
// key(v, id) = order(v) << 32 | (0xFFFFFFFF - id): a larger key ranks first,
// so the ranking "larger value, ties to the lower id" is a single unsigned
// compare.  The value and id are recovered exactly from the key (a -0 value
// comes back as +0; the two compare equal).  Key 0 is the empty slot.
#pragma once

#include "common.h"

namespace graft {

__device__ inline uint64_t rank_key(float v, int id) {
  return (static_cast<uint64_t>(float_order(v)) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(id));
}
__device__ inline float key_value(uint64_t key) {
  const uint32_t o = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ inline int key_id(uint64_t key) { return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key)); }

template <int K>
struct TopKeys {
  uint64_t k[K];
  __device__ void init() {
#pragma unroll
    for (int j = 0; j < K; ++j) k[j] = 0;
  }
  __device__ void insert(uint64_t x) {
    if (x <= k[K - 1]) return;
    k[K - 1] = x;
#pragma unroll
    for (int j = K - 1; j > 0; --j) {
      const uint64_t a = k[j - 1], b = k[j];
      const bool sw = b > a;
      k[j - 1] = sw ? b : a;
      k[j] = sw ? a : b;
    }
  }
  __device__ void pop_front() {
#pragma unroll
    for (int j = 0; j < K - 1; ++j) k[j] = k[j + 1];
    k[K - 1] = 0;
  }
};

// Largest key over the lanes of xor-groups of `width` lanes (width a power of
// two <= 64); every lane of the group gets the result.
__device__ inline uint64_t group_max(uint64_t x, int width) {
  for (int off = 1; off < width; off <<= 1) {
    const uint64_t o = __shfl_xor(x, off);
    x = o > x ? o : x;
  }
  return x;
}

// k rounds of extraction from the per-lane lists of one wavefront; lane j < k
// receives the j-th largest key.
template <int K>
__device__ inline uint64_t wave_extract(TopKeys<K> &L, int k) {
  const int lane = threadIdx.x & 63;
  uint64_t out = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t best = group_max(L.k[0], 64);
    if (L.k[0] == best) L.pop_front();
    if (lane == j) out = best;
  }
  return out;
}

}  // namespace graft
