// Tree-masked grouped-query attention of the flattened tree against the KV
// cache (Graft page, arXiv:2605.20104 write-up, section 2, third step: one
// parallel verification of the flattened tree with the rebuilt mask;
// TreeGraft page, section 3 and section 7 item 1: tree attention).
//
// Query row (node i, head h) sees cache slots 0..ctx-1 and tree slot ctx+j
// iff bit j of mask[i].  All N tree nodes times the G = Hq/Hkv heads of one
// KV head share every K/V tile, so one workgroup owns one (request, KV head,
// key split) and all of its N*G query rows: K/V are read from HBM once per
// split and staged through LDS, and both products run on MFMA:
//   S^T = K . Q^T   (A = K tile from LDS, B = Q fragments kept in registers)
//   O^T = V^T . P^T (A = V^T tile from LDS, B = P straight from the S^T
//                    accumulators, re-packed to bf16)
// Computing the transposes puts one query row per lane column in both
// accumulators, so the online-softmax statistics of a row live in one lane
// group and rescaling O needs no cross-lane traffic.  A V_MFMA_F32_16X16X32
// lane holds keys {4g..4g+3} and {16+4g..16+4g+3} of its row after the S^T
// step; the P^T operand uses exactly that key set, and the V^T fragment is
// read with the same set, so no shuffle is needed between the two products.
//
// The key range is split over workgroups (8 KV heads alone cannot fill 256
// CUs); each split writes unnormalised O, the running max and the exp-sum,
// and a merge kernel combines splits with the usual log-sum-exp weights.
// With a single split the workgroup normalises and writes bf16 directly.
#include <cmath>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int KCH = 32;      // keys per staged chunk (two 16-key MFMA blocks)
constexpr int MIN_SPLIT = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }
__device__ inline u32x4 load16(const graft_bf16 *p) { return *reinterpret_cast<const u32x4 *>(p); }

template <int D>
struct Smem {
  static constexpr int KSTR = D + 8;    // bf16 per K row (16 B pad)
  static constexpr int VSTR = KCH + 4;  // bf16 per V^T row (8 B pad)
  graft_bf16 k[KCH * KSTR];
  graft_bf16 vt[D * VSTR];
};

struct Params {
  int B, Hq, Hkv, G;
  float scale_log2;
  const graft_bf16 *q;
  const graft_bf16 *kc;
  const graft_bf16 *vc;
  const int64_t *kv_off;
  int64_t head_stride;
  const int32_t *ctx_len;
  int max_ctx;
  const int32_t *n;
  int max_n;
  const int32_t *row_off;
  const uint64_t *mask;
  int split_len, nsplit, rows_per_wg, row_groups, rows_cap;
  graft_bf16 *out;
  float *lse;
  float *ws_o;
  float *ws_ml;
  int32_t *err;
};

// Returns false (and flags once) when the request's lengths exceed the
// bounds the grid was sized for.
__device__ inline bool request_ok(const Params &P, int b, int &ctx, int &n) {
  ctx = P.ctx_len[b];
  n = P.n[b];
  const bool ok = ctx >= 0 && ctx <= P.max_ctx && n >= 1 && n <= P.max_n && n <= GRAFT_MAX_NODES &&
                  n <= P.row_off[b + 1] - P.row_off[b];
  if (!ok && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) graft::raise_flag(P.err, GRAFT_ERR_CAPACITY);
  return ok;
}

template <int D, int RBW>
__global__ __launch_bounds__(kThreads) void tree_attn_kernel(Params P) {
  constexpr int DS = D / 32;  // MFMA k-steps over the head dim
  constexpr int DB = D / 16;  // 16-wide output blocks over the head dim
  constexpr int PIECES = KCH * D / 8;
  __shared__ __attribute__((aligned(16))) Smem<D> sm;

  const int b = blockIdx.z;
  const int h = blockIdx.y / P.row_groups;
  const int rg = blockIdx.y - h * P.row_groups;
  const int split = blockIdx.x;
  int ctx, n;
  if (!request_ok(P, b, ctx, n)) return;
  const int L = ctx + n;
  const int k_begin = split * P.split_len;
  if (k_begin >= L) return;
  const int k_end = min(L, k_begin + P.split_len);
  const int rows_total = n * P.G;
  const int row_lo = rg * P.rows_per_wg;
  if (row_lo >= rows_total) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int r_off = P.row_off[b];

  // ---- this lane's query rows: Q fragments and tree-mask words
  bf16x8 qf[RBW][DS];
  uint64_t mrow[RBW];
  bool rvalid[RBW];
  bool active[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    const int rb0 = row_lo + (wave * RBW + j) * 16;
    active[j] = rb0 < rows_total;
    const int r = rb0 + l16;
    rvalid[j] = r < rows_total;
    const int node = r / P.G;
    const int hq = h * P.G + (r - node * P.G);
    mrow[j] = rvalid[j] ? P.mask[r_off + node] : 0ull;
    const graft_bf16 *qp = P.q + (static_cast<size_t>(r_off + node) * P.Hq + hq) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[j][s] = rvalid[j] ? __builtin_bit_cast(bf16x8, load16(qp + s * 32)) : zero8();
  }

  f32x4 oacc[RBW][DB];
  float m_run[RBW], l_run[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging: each thread moves one 16-byte piece of K and of V per chunk
  const bool stager = tid < PIECES;
  const int st_key = tid / (D / 8);
  const int st_col = tid - st_key * (D / 8);
  const size_t kv_base = static_cast<size_t>(P.kv_off[b]) + static_cast<size_t>(h) * P.head_stride;
  u32x4 kreg = u32x4{0u, 0u, 0u, 0u}, vreg = u32x4{0u, 0u, 0u, 0u};
  auto fetch = [&](int c0) {
    const int slot = c0 + st_key;
    if (stager && slot < k_end) {
      const size_t off = kv_base + static_cast<size_t>(slot) * D + st_col * 8;
      kreg = load16(P.kc + off);
      vreg = load16(P.vc + off);
    } else {
      kreg = u32x4{0u, 0u, 0u, 0u};
      vreg = u32x4{0u, 0u, 0u, 0u};
    }
  };
  fetch(k_begin);

  for (int c0 = k_begin; c0 < k_end; c0 += KCH) {
    __syncthreads();
    if (stager) {
      *reinterpret_cast<u32x4 *>(&sm.k[st_key * Smem<D>::KSTR + st_col * 8]) = kreg;
      // element e of the 16-byte piece is bits [16(e&1), 16(e&1)+16) of word e/2
      // (extracting lanes of a __bf16 vector here miscompiled: every lane read as lane 0)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sm.vt[(st_col * 8 + e) * Smem<D>::VSTR + st_key] =
            static_cast<graft_bf16>((vreg[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    }
    __syncthreads();
    if (c0 + KCH < k_end) fetch(c0 + KCH);

    // S^T blocks: sacc[j][kb][i] = S[row l16][key c0 + kb*16 + 4g + i]
    f32x4 sacc[RBW][2];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
      sacc[j][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sacc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sm.k[(kb * 16 + l16) * Smem<D>::KSTR + s * 32 + 8 * g]);
#pragma unroll
        for (int j = 0; j < RBW; ++j)
          if (active[j]) sacc[j][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[j][s], sacc[j][kb], 0, 0, 0);
      }
    }

    // online softmax (base 2) and P^T operands
    bf16x8 pb[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
      if (!active[j]) continue;
      float x[8];
      float cmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = c0 + kb * 16 + 4 * g + i;
          bool vis = key < k_end;
          if (vis && key >= ctx) vis = (mrow[j] >> (key - ctx)) & 1ull;
          const float v = vis ? sacc[j][kb][i] * P.scale_log2 : -INFINITY;
          x[kb * 4 + i] = v;
          cmax = fmaxf(cmax, v);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run[j], cmax);
      float alpha = 1.f;
      float psum = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run[j] - m_new);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = exp2f(x[e] - m_new);
          psum += x[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      m_run[j] = m_new;
      l_run[j] = l_run[j] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[j][db] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[j][e] = static_cast<__bf16>(x[e]);
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const graft_bf16 *vrow = &sm.vt[(db * 16 + l16) * Smem<D>::VSTR];
      const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow + 4 * g);
      const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 16 + 4 * g);
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
      for (int j = 0; j < RBW; ++j)
        if (active[j]) oacc[j][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[j], oacc[j][db], 0, 0, 0);
    }
  }

  // ---- epilogue: oacc[j][db][i] = O[row l16][d = db*16 + 4g + i]
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    if (!active[j]) continue;
    float l_tot = l_run[j];
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!rvalid[j]) continue;
    const int r = row_lo + (wave * RBW + j) * 16 + l16;
    if (P.nsplit == 1) {
      const int node = r / P.G;
      const int hq = h * P.G + (r - node * P.G);
      const size_t orow = static_cast<size_t>(r_off + node) * P.Hq + hq;
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = static_cast<__bf16>(oacc[j][db][i] * inv);
        *reinterpret_cast<bf16x4 *>(P.out + orow * D + db * 16 + 4 * g) = o;
      }
      if (P.lse && g == 0) P.lse[orow] = (m_run[j] + log2f(l_tot)) * kLn2;
    } else {
      const size_t slot = ((static_cast<size_t>(b) * P.Hkv + h) * P.nsplit + split) * P.rows_cap + r;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4 *>(P.ws_o + slot * D + db * 16 + 4 * g) = oacc[j][db];
      if (g == 0) {
        P.ws_ml[slot * 2] = m_run[j];
        P.ws_ml[slot * 2 + 1] = l_tot;
      }
    }
  }
}

// One thread per 4 output columns of one (request, KV head, query row).
template <int D>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(Params P) {
  constexpr int TPR = D / 4;         // threads per row
  constexpr int RPB = 256 / TPR;     // rows per block
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int r = blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 4;
  int ctx, n;
  if (!request_ok(P, b, ctx, n)) return;
  if (r >= n * P.G) return;
  const int L = ctx + n;
  const int ns = (L + P.split_len - 1) / P.split_len;
  const size_t base = (static_cast<size_t>(b) * P.Hkv + h) * P.nsplit * P.rows_cap + r;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, P.ws_ml[(base + static_cast<size_t>(s) * P.rows_cap) * 2]);
  float wsum = 0.f;
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; ++s) {
    const size_t slot = base + static_cast<size_t>(s) * P.rows_cap;
    const float ms = P.ws_ml[slot * 2];
    if (ms == -INFINITY) continue;
    const float wgt = exp2f(ms - M);
    wsum += wgt * P.ws_ml[slot * 2 + 1];
    o += wgt * *reinterpret_cast<const f32x4 *>(P.ws_o + slot * D + c);
  }
  const int node = r / P.G;
  const int hq = h * P.G + (r - node * P.G);
  const size_t orow = static_cast<size_t>(P.row_off[b] + node) * P.Hq + hq;
  const float inv = 1.f / wsum;
  bf16x4 ob;
#pragma unroll
  for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(o[i] * inv);
  *reinterpret_cast<bf16x4 *>(P.out + orow * D + c) = ob;
  if (P.lse && c == 0) P.lse[orow] = (M + log2f(wsum)) * kLn2;
}

struct Plan {
  int rbw, row_groups, rows_per_wg, rows_cap, split_len, nsplit;
  size_t ws_bytes;
};

Plan make_plan(int B, int Hq, int Hkv, int d, int max_ctx, int max_n) {
  Plan p{};
  const int G = Hq / Hkv;
  const int rows = max_n * G;
  const int rb = (rows + 15) / 16;
  // at most 3 row blocks per wave: 4 spills registers at d = 128
  if (rb <= kWaves) p.rbw = 1;
  else if (rb <= 2 * kWaves) p.rbw = 2;
  else p.rbw = 3;
  p.rows_per_wg = kWaves * p.rbw * 16;
  p.row_groups = (rows + p.rows_per_wg - 1) / p.rows_per_wg;
  p.rows_cap = rb * 16;
  const long long L = static_cast<long long>(max_ctx) + max_n;
  const long long units = static_cast<long long>(B) * Hkv * p.row_groups;
  long long want = units > 0 ? (512 + units - 1) / units : 1;
  if (want < 1) want = 1;
  long long len = (L + want - 1) / want;
  len = (len + KCH - 1) / KCH * KCH;
  if (len < MIN_SPLIT) len = MIN_SPLIT;
  p.split_len = static_cast<int>(len);
  p.nsplit = static_cast<int>((L + len - 1) / len);
  p.ws_bytes = p.nsplit > 1 ? static_cast<size_t>(B) * Hkv * p.nsplit * p.rows_cap * (d + 2) * sizeof(float) : 0;
  return p;
}

bool shape_ok(int B, int Hq, int Hkv, int d, int max_ctx, int max_n) {
  return B >= 0 && Hkv > 0 && Hq > 0 && Hq % Hkv == 0 && Hq / Hkv <= 16 && (d == 64 || d == 128) &&
         max_ctx >= 0 && max_n >= 1 && max_n <= GRAFT_MAX_NODES;
}

template <int D>
void launch(const Plan &pl, const Params &P, dim3 grid, hipStream_t s) {
  switch (pl.rbw) {
    case 1: hipLaunchKernelGGL((tree_attn_kernel<D, 1>), grid, dim3(kThreads), 0, s, P); break;
    case 2: hipLaunchKernelGGL((tree_attn_kernel<D, 2>), grid, dim3(kThreads), 0, s, P); break;
    default: hipLaunchKernelGGL((tree_attn_kernel<D, 3>), grid, dim3(kThreads), 0, s, P); break;
  }
  if (pl.nsplit > 1) {
    constexpr int RPB = 256 / (D / 4);
    dim3 mg((pl.rows_cap + RPB - 1) / RPB, P.Hkv, P.B);
    hipLaunchKernelGGL(tree_attn_merge_kernel<D>, mg, dim3(256), 0, s, P);
  }
}

}  // namespace

extern "C" size_t graft_tree_attention_workspace_bytes(int B, int Hq, int Hkv, int d, int max_ctx, int max_n) {
  if (!shape_ok(B, Hq, Hkv, d, max_ctx, max_n) || B == 0) return 0;
  return make_plan(B, Hq, Hkv, d, max_ctx, max_n).ws_bytes;
}

extern "C" int graft_tree_attention(int B, int Hq, int Hkv, int d, float scale, const graft_bf16 *q,
                                    const graft_bf16 *kcache, const graft_bf16 *vcache, const int64_t *kv_off,
                                    int64_t kv_head_stride, const int32_t *ctx_len, int max_ctx,
                                    const int32_t *n, int max_n, const int32_t *row_off, const uint64_t *mask,
                                    graft_bf16 *out, float *lse, void *ws, size_t ws_bytes, int32_t *err_flag,
                                    graft_stream stream) {
  using graft::fail;
  if (!shape_ok(B, Hq, Hkv, d, max_ctx, max_n)) {
    if (d != 64 && d != 128 && d > 0) return fail(GRAFT_EUNSUPPORTED, "tree_attention: head dim %d (built: 64, 128)", d);
    return fail(GRAFT_EINVAL, "tree_attention: B=%d Hq=%d Hkv=%d d=%d max_ctx=%d max_n=%d", B, Hq, Hkv, d, max_ctx,
                max_n);
  }
  if (B == 0) return GRAFT_OK;
  if (!q || !kcache || !vcache || !kv_off || !ctx_len || !n || !row_off || !mask || !out)
    return fail(GRAFT_EINVAL, "tree_attention: NULL array");
  if (kv_head_stride < static_cast<int64_t>(max_ctx + max_n) * d)
    return fail(GRAFT_EINVAL, "tree_attention: kv_head_stride %lld < (max_ctx + max_n) * d",
                static_cast<long long>(kv_head_stride));
  const Plan pl = make_plan(B, Hq, Hkv, d, max_ctx, max_n);
  if (ws_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && !ws))
    return fail(GRAFT_EINVAL, "tree_attention: workspace %zu bytes < %zu", ws_bytes, pl.ws_bytes);
  if (pl.nsplit > 65535 || static_cast<long long>(Hkv) * pl.row_groups > 65535 || B > 65535)
    return fail(GRAFT_EINVAL, "tree_attention: grid too large");
  graft::clear_error();
  Params P{};
  P.B = B;
  P.Hq = Hq;
  P.Hkv = Hkv;
  P.G = Hq / Hkv;
  P.scale_log2 = scale * kLog2e;
  P.q = q;
  P.kc = kcache;
  P.vc = vcache;
  P.kv_off = kv_off;
  P.head_stride = kv_head_stride;
  P.ctx_len = ctx_len;
  P.max_ctx = max_ctx;
  P.n = n;
  P.max_n = max_n;
  P.row_off = row_off;
  P.mask = mask;
  P.split_len = pl.split_len;
  P.nsplit = pl.nsplit;
  P.rows_per_wg = pl.rows_per_wg;
  P.row_groups = pl.row_groups;
  P.rows_cap = pl.rows_cap;
  P.out = out;
  P.lse = lse;
  P.ws_o = static_cast<float *>(ws);
  P.ws_ml = pl.ws_bytes ? P.ws_o + static_cast<size_t>(B) * Hkv * pl.nsplit * pl.rows_cap * d : nullptr;
  P.err = err_flag;
  dim3 grid(pl.nsplit, Hkv * pl.row_groups, B);
  hipStream_t s = graft::as_stream(stream);
  if (d == 128) launch<128>(pl, P, grid, s);
  else launch<64>(pl, P, grid, s);
  return graft::check_launch("tree_attention");
}
