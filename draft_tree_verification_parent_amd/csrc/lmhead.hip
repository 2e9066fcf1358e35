// lm-head GEMM: logits[m, v] = sum_h hidden[m, h] * W[v, h], bf16 in, fp32 out,
// optionally fused with the per-row top-k so the logits never reach HBM.
//
// The verification pass ends in each tree position's next-token
// distribution, which the table update and the acceptance test read (Graft
// page, arXiv:2605.20104 write-up, section 2, third step).
//
// With M = tree nodes (tens) and V x H = 0.5-0.8 G weights, this is a
// weight-streaming product bound by HBM (about 60 flop per weight byte).
// Each workgroup owns BV = 32 * WAVES vocabulary rows and BM = 64 hidden rows:
//  * W is read once, straight from HBM into MFMA A-operand registers
//    (16 contiguous bytes per lane); the next K chunk's loads are issued
//    before the current chunk's MFMAs;
//  * the hidden states, shared by every workgroup, are staged through a
//    double-buffered LDS tile in K chunks of 256 and read as B operands; the
//    next chunk's hidden loads are issued *before* the next W loads, so that
//    waiting for them (vector-memory counters retire in order) never waits
//    for W;
//  * V_MFMA_F32_16X16X32_BF16 computes 16 vocabulary rows x 16 hidden rows;
//    each lane ends with 4 consecutive vocabulary entries of one row.
// Fused top-k: the 64 x BV logit tile goes through LDS, WAVES threads per row
// each rank 32 entries into a sorted register list, the lists of a row are
// merged with xor shuffles, and k (value, id) candidates per (row, tile) are
// written; a second kernel merges the tiles (same (value desc, id asc)
// order, so the result does not depend on the split).
// Tiles are ordered so that the M tiles of one V tile are consecutive on one
// XCD (workgroups are dealt round-robin to the 8 XCDs), which keeps repeated
// W tiles in that XCD's L2 when M > 64.
#include <climits>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "topk_list.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBV = kWaves * 32;

__device__ inline bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ inline u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

template <int KC, bool FUSED, int K>
__global__ __launch_bounds__(kThreads, 4) void lmhead_kernel(int M, int H, int V, int k,
                                                           const graft_bf16 *__restrict__ hidden,
                                                           const graft_bf16 *__restrict__ w,
                                                           float *__restrict__ logits,
                                                           uint64_t *__restrict__ part_out, int tiles_m,
                                                           int tiles_v) {
  constexpr int WAVES = kWaves;
  constexpr int BV = kBV;
  constexpr int STR = KC + 8;             // bf16 per staged hidden row (16 B pad)
  constexpr int KS = KC / 32;             // MFMA k-steps per chunk
  constexpr int PPT = BM * KC / 8 / kThreads;  // hidden 16-byte pieces staged per thread
  constexpr int TSTR = BV + 4;            // floats per row of the fused top-k logit tile
  constexpr int STAGE_BYTES = 2 * BM * STR * 2;
  constexpr int TILE_BYTES = FUSED ? BM * TSTR * 4 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGE_BYTES > TILE_BYTES ? STAGE_BYTES : TILE_BYTES];
  graft_bf16(*s_h)[BM * STR] = reinterpret_cast<graft_bf16(*)[BM * STR]>(smem);

  const int total = tiles_m * tiles_v;
  const int per_xcd = (total + 7) / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total) return;
  const int tm = logical % tiles_m;
  const int tv = logical / tiles_m;
  const int m0 = tm * BM;
  const int v0 = tv * BV;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // Every load below is unconditional: rows past V (or M) read the last valid
  // row and their outputs are never stored or ranked.  (Conditional loads
  // compile to branches whose joins drain the memory pipeline.)
  const graft_bf16 *wp[2];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) {
    const int r = v0 + wave * 32 + vb * 16 + l16;
    wp[vb] = w + static_cast<size_t>(r < V ? r : V - 1) * H + 8 * g;
  }
  // hidden staging: thread owns 16-byte column hcol of rows hrow0 + t * (kThreads / (KC / 8))
  constexpr int ROWS_PER_PASS = kThreads / (KC / 8);
  const int hcol = tid % (KC / 8);
  const int hrow0 = tid / (KC / 8);
  const graft_bf16 *hbase = hidden + hcol * 8;
  const int hd0 = hrow0 * STR + hcol * 8;

  f32x4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wa[2][KS], wb[2][KS], hr[PPT];
  auto load_w = [&](u32x4 (&d)[2][KS], int c) {
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        d[vb][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wp[vb] + c * KC + s * 32));
  };
  auto load_h = [&](int c) {
#pragma unroll
    for (int t = 0; t < PPT; ++t) {
      const int m = min(m0 + hrow0 + t * ROWS_PER_PASS, M - 1);
      hr[t] = *reinterpret_cast<const u32x4 *>(hbase + static_cast<size_t>(m) * H + c * KC);
    }
  };
  auto store_h = [&](int buf) {
#pragma unroll
    for (int t = 0; t < PPT; ++t)
      *reinterpret_cast<u32x4 *>(&s_h[buf][hd0 + t * ROWS_PER_PASS * STR]) = hr[t];
  };
  auto compute = [&](const u32x4 (&d)[2][KS], int buf) {
    const graft_bf16 *hb = s_h[buf];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 bh[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        bh[mb] = *reinterpret_cast<const bf16x8 *>(&hb[(mb * 16 + l16) * STR + s * 32 + 8 * g]);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[vb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(d[vb][s]), bh[mb], acc[vb][mb], 0, 0, 0);
    }
  };

  // Two W register buffers used in strict ping-pong (the loop is unrolled by
  // two), so no register copy of an in-flight load ever forces a full wait.
  const int nch = H / KC;
  load_h(0);
  load_w(wa, 0);
  store_h(0);
  __syncthreads();
  for (int c = 0; c + 1 < nch; c += 2) {
    load_h(c + 1);
    load_w(wb, c + 1);
    __builtin_amdgcn_sched_barrier(0x38F);  // keep these loads ahead of the MFMAs
    compute(wa, 0);
    store_h(1);
    __syncthreads();
    const int c2 = c + 2 < nch ? c + 2 : c + 1;
    load_h(c2);
    load_w(wa, c2);
    __builtin_amdgcn_sched_barrier(0x38F);
    compute(wb, 1);
    store_h(0);
    __syncthreads();
  }
  if (nch & 1) {
    compute(wa, 0);
    __syncthreads();
  }

  // lane holds logit[m0 + mb*16 + l16][v0 + wave*32 + vb*16 + 4g + i]
  if constexpr (!FUSED) {
    const bool vec = (V & 3) == 0;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + mb * 16 + l16;
      if (m >= M) continue;
      float *row = logits + static_cast<size_t>(m) * V;
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        const int v = v0 + wave * 32 + vb * 16 + 4 * g;
        const f32x4 r = acc[vb][mb];
        if (vec && v < V) {
          *reinterpret_cast<float4 *>(row + v) = make_float4(r[0], r[1], r[2], r[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v + i < V) row[v + i] = r[i];
        }
      }
    }
  } else {
    float *s_t = reinterpret_cast<float *>(smem);
    // (the last barrier above ordered every read of s_h before this)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        const int vloc = wave * 32 + vb * 16 + 4 * g;
        *reinterpret_cast<f32x4 *>(&s_t[(mb * 16 + l16) * TSTR + vloc]) = acc[vb][mb];
      }
    __syncthreads();
    // WAVES consecutive threads per row, 32 entries each
    const int row = tid / WAVES;
    const int part = tid - row * WAVES;
    const int m = m0 + row;
    graft::TopKeys<K> L;
    L.init();
    const int vbase = v0 + part * 32;
#pragma unroll 8
    for (int j = 0; j < 32; ++j)
      if (vbase + j < V) L.insert(graft::rank_key(s_t[row * TSTR + part * 32 + j], vbase + j));
    for (int j = 0; j < k; ++j) {
      const uint64_t best = graft::group_max(L.k[0], WAVES);
      if (L.k[0] == best) L.pop_front();
      if (part == 0 && m < M) part_out[(static_cast<size_t>(m) * tiles_v + tv) * k + j] = best;
    }
  }
}

}  // namespace

namespace graft {
size_t lmhead_fused_ws_bytes(int M, int V, int k) {
  const int tiles_v = (V + kBV - 1) / kBV;
  return static_cast<size_t>(M) * tiles_v * k * sizeof(uint64_t);
}
}  // namespace graft

extern "C" size_t graft_lmhead_topk_workspace_bytes(int M, int V, int k) {
  if (M <= 0 || V <= 0 || k <= 0) return 0;
  const size_t a = graft::topk_plan(M, V, k).ws_bytes;
  const size_t b = graft::lmhead_fused_ws_bytes(M, V, k);
  return a > b ? a : b;
}

extern "C" int graft_lmhead_topk(int M, int H, int V, int k, const graft_bf16 *hidden, const graft_bf16 *w,
                                 float *logits, int32_t *topk_id, float *topk_val, void *ws,
                                 size_t ws_bytes, graft_stream stream) {
  using graft::fail;
  if (M < 0 || V <= 0 || k < 0 || k > GRAFT_MAX_K || k > V)
    return fail(GRAFT_EINVAL, "lmhead_topk: M=%d V=%d k=%d", M, V, k);
  if (hidden && (H <= 0 || H % 64 != 0))
    return fail(GRAFT_EINVAL, "lmhead_topk: H=%d must be a positive multiple of 64", H);
  if (!hidden && !logits) return fail(GRAFT_EINVAL, "lmhead_topk: both hidden and logits are NULL");
  if (hidden && !w) return fail(GRAFT_EINVAL, "lmhead_topk: W is NULL");
  if (!logits && k == 0) return fail(GRAFT_EINVAL, "lmhead_topk: fused mode needs k > 0");
  if (!hidden && k == 0) return fail(GRAFT_EINVAL, "lmhead_topk: nothing to do (no hidden, k = 0)");
  if (k > 0 && !topk_id) return fail(GRAFT_EINVAL, "lmhead_topk: topk_id is NULL");
  if (M == 0) return GRAFT_OK;
  const bool fused = hidden && !logits;
  const size_t need = fused ? graft::lmhead_fused_ws_bytes(M, V, k) : (k > 0 ? graft::topk_plan(M, V, k).ws_bytes : 0);
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(GRAFT_EINVAL, "lmhead_topk: workspace %zu bytes < %zu", ws_bytes, need);
  graft::clear_error();
  hipStream_t s = graft::as_stream(stream);
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_v = (V + kBV - 1) / kBV;
  const int grid = (tiles_m * tiles_v + 7) / 8 * 8;
  // K chunk of 128 hidden columns when it divides H (the common case), else 64
  const bool kc128 = H % 128 == 0;
  auto launch = [&](auto kc_tag, auto fused_tag, auto k_tag, uint64_t *pk) {
    constexpr int KCv = decltype(kc_tag)::value;
    constexpr bool F = decltype(fused_tag)::value;
    constexpr int Kv = decltype(k_tag)::value;
    hipLaunchKernelGGL((lmhead_kernel<KCv, F, Kv>), dim3(grid), dim3(kThreads), 0, s, M, H, V, F ? k : 0, hidden, w,
                       F ? nullptr : logits, pk, tiles_m, tiles_v);
  };
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using I8 = std::integral_constant<int, 8>;
  using I16 = std::integral_constant<int, 16>;
  using T = std::true_type;
  using Fz = std::false_type;
  if (fused) {
    uint64_t *pk = static_cast<uint64_t *>(ws);
    if (kc128 && k <= 8) launch(I128{}, T{}, I8{}, pk);
    else if (kc128) launch(I128{}, T{}, I16{}, pk);
    else if (k <= 8) launch(I64{}, T{}, I8{}, pk);
    else launch(I64{}, T{}, I16{}, pk);
    int rc = graft::check_launch("lmhead (fused top-k)");
    if (rc != GRAFT_OK) return rc;
    return graft::launch_topk_merge(M, tiles_v, k, pk, topk_id, topk_val, s);
  }
  if (hidden) {
    if (kc128) launch(I128{}, Fz{}, I8{}, nullptr);
    else launch(I64{}, Fz{}, I8{}, nullptr);
    int rc = graft::check_launch("lmhead");
    if (rc != GRAFT_OK) return rc;
  }
  if (k > 0) return graft::launch_topk(M, V, k, logits, topk_id, topk_val, ws, s);
  return GRAFT_OK;
}
