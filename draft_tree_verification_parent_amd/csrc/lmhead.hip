// lm-head GEMM: logits[m, v] = sum_h hidden[m, h] * W[v, h], bf16 in, fp32 out.
//
// The verification pass ends in each tree position's next-token
// distribution, which the table update and the acceptance test read (Graft
// page, arXiv:2605.20104 write-up, section 2, third step).
//
// With M = tree nodes (tens) and V x H = 0.5-0.8 G weights, this is a
// weight-streaming product bound by HBM (about 60 flop per weight byte).
// Each workgroup owns BV = 128 vocabulary rows and BM = 64 hidden rows:
//  * W is read once, straight from HBM into MFMA A-operand registers
//    (16 contiguous bytes per lane), with the next K chunk's loads issued
//    before the current chunk's MFMAs;
//  * the hidden states, shared by every workgroup, are staged through LDS in
//    K chunks of 256 and read as MFMA B operands;
//  * V_MFMA_F32_16X16X32_BF16 computes 16 vocabulary rows x 16 hidden rows;
//    each lane ends with 4 consecutive vocabulary entries of one row and
//    writes them as one float4.
// Tiles are ordered so that the M tiles of one V tile are consecutive on one
// XCD (workgroups are dealt round-robin to the 8 XCDs), which keeps repeated
// W tiles in that XCD's L2 when M > 64.
#include "common.h"
#include "kernels.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = 64;
constexpr int BV = 128;
constexpr int KC = 256;
constexpr int KS = KC / 32;          // MFMA k-steps per chunk
constexpr int LDS_STRIDE = KC + 8;   // bf16 per staged row: 16 B pad against bank conflicts

__device__ inline bf16x8 load16(const graft_bf16 *p) {
  const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return __builtin_bit_cast(bf16x8, u);
}
__device__ inline bf16x8 load16_cached(const graft_bf16 *p) {
  const u32x4 u = *reinterpret_cast<const u32x4 *>(p);
  return __builtin_bit_cast(bf16x8, u);
}
__device__ inline bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

__device__ inline void load_w_chunk(bf16x8 (&dst)[2][KS], const graft_bf16 *w0, const graft_bf16 *w1,
                                    bool ok0, bool ok1, int k0, int kc) {
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (s * 32 < kc) {
      const bf16x8 a = load16(w0 + k0 + s * 32);
      const bf16x8 b = load16(w1 + k0 + s * 32);
      dst[0][s] = ok0 ? a : zero8();
      dst[1][s] = ok1 ? b : zero8();
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void lmhead_kernel(int M, int H, int V,
                                                             const graft_bf16 *__restrict__ hidden,
                                                             const graft_bf16 *__restrict__ w,
                                                             float *__restrict__ logits, int tiles_m,
                                                             int tiles_v) {
  __shared__ __attribute__((aligned(16))) graft_bf16 s_h[BM * LDS_STRIDE];

  const int total = tiles_m * tiles_v;
  const int per_xcd = (total + 7) / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total) return;
  const int m0 = (logical % tiles_m) * BM;
  const int v0 = (logical / tiles_m) * BV;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  const int vr0 = v0 + wave * 32 + l16;
  const int vr1 = vr0 + 16;
  const bool ok0 = vr0 < V;
  const bool ok1 = vr1 < V;
  const graft_bf16 *w0 = w + static_cast<size_t>(ok0 ? vr0 : 0) * H + 8 * g;
  const graft_bf16 *w1 = w + static_cast<size_t>(ok1 ? vr1 : 0) * H + 8 * g;

  f32x4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (H + KC - 1) / KC;
  bf16x8 wc[2][KS];
  load_w_chunk(wc, w0, w1, ok0, ok1, 0, H < KC ? H : KC);

  for (int c = 0; c < nchunks; ++c) {
    const int k0 = c * KC;
    const int kc = H - k0 < KC ? H - k0 : KC;
    const int pieces = kc / 8;  // 16-byte pieces per staged row

    __syncthreads();
    for (int p = tid; p < BM * pieces; p += kThreads) {
      const int row = p / pieces;
      const int col = p - row * pieces;
      const int m = m0 + row;
      const bf16x8 x = m < M ? load16_cached(hidden + static_cast<size_t>(m) * H + k0 + col * 8) : zero8();
      *reinterpret_cast<bf16x8 *>(&s_h[row * LDS_STRIDE + col * 8]) = x;
    }
    __syncthreads();

    bf16x8 wn[2][KS];
    if (c + 1 < nchunks) {
      const int kn = H - (k0 + KC) < KC ? H - (k0 + KC) : KC;
      load_w_chunk(wn, w0, w1, ok0, ok1, k0 + KC, kn);
    }

#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s * 32 < kc) {
        bf16x8 bh[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          bh[mb] = *reinterpret_cast<const bf16x8 *>(&s_h[(mb * 16 + l16) * LDS_STRIDE + s * 32 + 8 * g]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          acc[0][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wc[0][s], bh[mb], acc[0][mb], 0, 0, 0);
          acc[1][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wc[1][s], bh[mb], acc[1][mb], 0, 0, 0);
        }
      }
    }
    if (c + 1 < nchunks) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        wc[0][s] = wn[0][s];
        wc[1][s] = wn[1][s];
      }
    }
  }

  // lane holds logits[m0 + mb*16 + l16][v0 + wave*32 + vb*16 + 4g + i]
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
}

}  // namespace

extern "C" size_t graft_lmhead_topk_workspace_bytes(int M, int V, int k) {
  if (M <= 0 || V <= 0 || k <= 0) return 0;
  return graft::topk_plan(M, V, k).ws_bytes;
}

extern "C" int graft_lmhead_topk(int M, int H, int V, int k, const graft_bf16 *hidden, const graft_bf16 *w,
                                 float *logits, int32_t *topk_id, float *topk_val, void *ws,
                                 size_t ws_bytes, graft_stream stream) {
  using graft::fail;
  if (M < 0 || V <= 0 || k < 0 || k > GRAFT_MAX_K || k > V)
    return fail(GRAFT_EINVAL, "lmhead_topk: M=%d V=%d k=%d", M, V, k);
  if (hidden && (H <= 0 || H % 64 != 0)) return fail(GRAFT_EINVAL, "lmhead_topk: H=%d must be a positive multiple of 64", H);
  if (!logits) {
    if (hidden) return fail(GRAFT_EUNSUPPORTED, "lmhead_topk: fused mode (logits NULL) is not built");
    return fail(GRAFT_EINVAL, "lmhead_topk: both hidden and logits are NULL");
  }
  if (hidden && !w) return fail(GRAFT_EINVAL, "lmhead_topk: W is NULL");
  if (!hidden && k == 0) return fail(GRAFT_EINVAL, "lmhead_topk: nothing to do (no hidden, k = 0)");
  if (k > 0 && !topk_id) return fail(GRAFT_EINVAL, "lmhead_topk: topk_id is NULL");
  if (M == 0) return GRAFT_OK;
  const size_t need = k > 0 ? graft::topk_plan(M, V, k).ws_bytes : 0;
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(GRAFT_EINVAL, "lmhead_topk: workspace %zu bytes < %zu", ws_bytes, need);
  graft::clear_error();
  hipStream_t s = graft::as_stream(stream);
  if (hidden) {
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_v = (V + BV - 1) / BV;
    const int total = tiles_m * tiles_v;
    const int grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL(lmhead_kernel, dim3(grid), dim3(kThreads), 0, s, M, H, V, hidden, w, logits, tiles_m,
                       tiles_v);
    int rc = graft::check_launch("lmhead");
    if (rc != GRAFT_OK) return rc;
  }
  if (k > 0) return graft::launch_topk(M, V, k, logits, topk_id, topk_val, ws, s);
  return GRAFT_OK;
}
