// Per-thread sorted top-K lists over (value desc, id asc), as 64-bit keys.
//
// key(v, id) = order(v) << 32 | (0xFFFFFFFF - id): a larger key ranks first,
// so the ranking "larger value, ties to the lower id" is a single unsigned
// compare.  The value and id are recovered exactly from the key (a -0 value
// comes back as +0; the two compare equal).  Key 0 is the empty slot.
#pragma once

#include <cmath>
#include <type_traits>

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

// A sorted list of K (value, id) keys whose compare-exchanges are two
// fp64 instructions.  Key bits: order(value) << 30 | (2^30 - 1 - id): the
// top two bits are clear, so as an fp64 bit pattern every key is a finite
// non-negative number (subnormal for the smallest orders; fp64 subnormals
// are not flushed) and fp64 order equals the integer order of the bits, the
// (value desc, id asc) ranking.  0.0 is the empty slot.  Ids below 2^30 - 1.
template <int K>
struct F64Keys {
  double k[K];
  __device__ void init() {
#pragma unroll
    for (int j = 0; j < K; ++j) k[j] = 0.0;
  }
  __device__ static double make(float v, int id) {
    const uint64_t bits = (static_cast<uint64_t>(graft::float_order(v)) << 30) |
                          static_cast<uint64_t>((1u << 30) - 1u - static_cast<uint32_t>(id));
    return __longlong_as_double(static_cast<long long>(bits));
  }
  // the K-th key's value (-inf while the list has an empty slot)
  __device__ float kth_value() const {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(k[K - 1]));
    return b == 0 ? -INFINITY : graft::key_value(static_cast<uint64_t>(static_cast<uint32_t>(b >> 30)) << 32);
  }
  // branch-free insertion: x bubbles down the descending list (0.0, the
  // empty key, leaves it unchanged).  One v_max_f64 and one v_min_f64 per
  // slot, written out: the library calls would add two canonicalising
  // operations each, and no key is a NaN.
  __device__ void insert(double x) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      double hi, lo;
      asm("v_max_f64 %0, %2, %3\n\tv_min_f64 %1, %2, %3" : "=&v"(hi), "=&v"(lo) : "v"(k[j]), "v"(x));
      k[j] = hi;
      x = lo;
    }
  }
  // the order of the head (largest) key's value, 0 while the list is empty
  __device__ uint32_t head_order() const {
    return static_cast<uint32_t>(static_cast<uint64_t>(__double_as_longlong(k[0])) >> 30);
  }
  // the key of slot j in the rank_key format the merge reads (0 = empty)
  __device__ uint64_t rank_key(int j) const {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(k[j]));
    if (b == 0) return 0;
    const uint32_t id = (1u << 30) - 1u - static_cast<uint32_t>(b & ((1u << 30) - 1u));
    return (static_cast<uint64_t>(static_cast<uint32_t>(b >> 30)) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - id);
  }
};

// 32-bit lane exchanges without LDS: DPP within a row of 16 lanes, the
// gfx950 row-swap permutes across rows.  Every lane of a group ends up
// paired with a lane of the other half of its group, which is all a
// max-reduction needs.
namespace lanes {
constexpr int kXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141; // lane i <-> 7 - i within 8 lanes
constexpr int kMirror = 0x140;     // lane i <-> 15 - i within 16 lanes
template <int CTRL>
__device__ inline uint32_t dpp(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}
}  // namespace lanes

__device__ inline uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Largest key over aligned groups of W lanes (W a power of two <= 64); every
// lane of the group gets the result.
template <int W>
__device__ inline uint64_t group_max(uint64_t x) {
  auto step_dpp = [](uint64_t v, auto ctrl_tag) {
    constexpr int C = decltype(ctrl_tag)::value;
    const uint32_t lo = lanes::dpp<C>(static_cast<uint32_t>(v));
    const uint32_t hi = lanes::dpp<C>(static_cast<uint32_t>(v >> 32));
    return max_u64(v, (static_cast<uint64_t>(hi) << 32) | lo);
  };
  if constexpr (W >= 2) x = step_dpp(x, std::integral_constant<int, lanes::kXor1>{});
  if constexpr (W >= 4) x = step_dpp(x, std::integral_constant<int, lanes::kXor2>{});
  if constexpr (W >= 8) x = step_dpp(x, std::integral_constant<int, lanes::kHalfMirror>{});
  if constexpr (W >= 16) x = step_dpp(x, std::integral_constant<int, lanes::kMirror>{});
  if constexpr (W >= 32) {
    const auto lo = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
    const auto hi =
        __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x >> 32), static_cast<uint32_t>(x >> 32), false, false);
    x = max_u64((static_cast<uint64_t>(hi[0]) << 32) | lo[0], (static_cast<uint64_t>(hi[1]) << 32) | lo[1]);
  }
  if constexpr (W >= 64) {
    const auto lo = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
    const auto hi =
        __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x >> 32), static_cast<uint32_t>(x >> 32), false, false);
    x = max_u64((static_cast<uint64_t>(hi[0]) << 32) | lo[0], (static_cast<uint64_t>(hi[1]) << 32) | lo[1]);
  }
  return x;
}

// Largest 32-bit value over the 64 lanes of a wavefront (every lane gets it).
__device__ inline uint32_t wave_max_u32(uint32_t x) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  x = mx(x, lanes::dpp<lanes::kXor1>(x));
  x = mx(x, lanes::dpp<lanes::kXor2>(x));
  x = mx(x, lanes::dpp<lanes::kHalfMirror>(x));
  x = mx(x, lanes::dpp<lanes::kMirror>(x));
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = mx(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return mx(b[0], b[1]);
}

// Value of the lane whose index differs from this lane's in bit J, without
// LDS traffic: DPP quad permutes (J = 1, 2), DPP row rotates (J = 4, 8;
// lane i reads lane i - N mod 16 under a rotate by N) and the gfx950
// row-swap permutes (J = 16, 32), which hand back the even and the odd
// half of each pair of rows.
template <int J>
__device__ inline uint32_t lane_xor32(uint32_t x, int lane) {
  const int v = static_cast<int>(x);
  if constexpr (J == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  } else if constexpr (J == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  } else if constexpr (J == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, v, 0x12C, 0xF, 0xF, false);  // lane i + 4
    const int dn = __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);  // lane i - 4
    return static_cast<uint32_t>((lane & 4) ? dn : up);
  } else if constexpr (J == 8) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane distance 1..32");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

// The K-th largest of the 64 lanes' values (0 = none): a bitonic sort of the
// 64 values, largest in lane 0, then lane K - 1's value, in 21 exchange
// steps whatever K (K rounds of a wave-wide maximum cost about 7 per round).
template <int K>
__device__ inline uint32_t wave_kth_u32(uint32_t v) {
  static_assert(K >= 1 && K <= 64, "one value per lane");
  const int lane = static_cast<int>(threadIdx.x & 63);
  auto step = [&](auto k_tag, auto j_tag) {
    constexpr int KB = decltype(k_tag)::value;
    constexpr int J = decltype(j_tag)::value;
    const uint32_t y = lane_xor32<J>(v, lane);
    // descending overall: within blocks of KB whose bit KB is clear the
    // lower lane of each pair keeps the larger value
    const bool keep_max = ((lane & KB) == 0) == ((lane & J) == 0);
    v = keep_max ? (v > y ? v : y) : (v < y ? v : y);
  };
  using std::integral_constant;
  step(integral_constant<int, 2>{}, integral_constant<int, 1>{});
  step(integral_constant<int, 4>{}, integral_constant<int, 2>{});
  step(integral_constant<int, 4>{}, integral_constant<int, 1>{});
  step(integral_constant<int, 8>{}, integral_constant<int, 4>{});
  step(integral_constant<int, 8>{}, integral_constant<int, 2>{});
  step(integral_constant<int, 8>{}, integral_constant<int, 1>{});
  step(integral_constant<int, 16>{}, integral_constant<int, 8>{});
  step(integral_constant<int, 16>{}, integral_constant<int, 4>{});
  step(integral_constant<int, 16>{}, integral_constant<int, 2>{});
  step(integral_constant<int, 16>{}, integral_constant<int, 1>{});
  step(integral_constant<int, 32>{}, integral_constant<int, 16>{});
  step(integral_constant<int, 32>{}, integral_constant<int, 8>{});
  step(integral_constant<int, 32>{}, integral_constant<int, 4>{});
  step(integral_constant<int, 32>{}, integral_constant<int, 2>{});
  step(integral_constant<int, 32>{}, integral_constant<int, 1>{});
  step(integral_constant<int, 64>{}, integral_constant<int, 32>{});
  step(integral_constant<int, 64>{}, integral_constant<int, 16>{});
  step(integral_constant<int, 64>{}, integral_constant<int, 8>{});
  step(integral_constant<int, 64>{}, integral_constant<int, 4>{});
  step(integral_constant<int, 64>{}, integral_constant<int, 2>{});
  step(integral_constant<int, 64>{}, integral_constant<int, 1>{});
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), K - 1));
}

// Largest float over aligned groups of W <= 8 lanes (every lane of the group gets it).
template <int W>
__device__ inline float group_maxf(float x) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8, "groups of 1, 2, 4 or 8 lanes");
  if constexpr (W >= 2) x = fmaxf(x, __uint_as_float(lanes::dpp<lanes::kXor1>(__float_as_uint(x))));
  if constexpr (W >= 4) x = fmaxf(x, __uint_as_float(lanes::dpp<lanes::kXor2>(__float_as_uint(x))));
  if constexpr (W >= 8) x = fmaxf(x, __uint_as_float(lanes::dpp<lanes::kHalfMirror>(__float_as_uint(x))));
  return x;
}

// k rounds of extraction from the per-lane lists of one wavefront; lane j < k
// receives the j-th largest key.
template <int K>
__device__ inline uint64_t wave_extract(TopKeys<K> &L, int k) {
  const int lane = threadIdx.x & 63;
  uint64_t out = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t best = group_max<64>(L.k[0]);
    if (L.k[0] == best) L.pop_front();
    if (lane == j) out = best;
  }
  return out;
}

}  // namespace graft
