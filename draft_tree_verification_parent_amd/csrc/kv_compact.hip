// KV compaction and round chaining.
//
// The flattened tree is verified in one pass and only the accepted output
// is kept; the next round drafts from the bonus token (Graft page, section
// 2, third step).  The tree's K/V rows sit at cache slots ctx .. ctx+n-1 in
// flattened order, so the accepted path root, p1, .., pa moves to slots
// ctx .. ctx+a (what decoding those tokens one at a time would have
// written), the context grows by a+1 and the bonus token becomes the root.
//
// One workgroup per (KV head, layer, request): at most 63 K rows and 63 V
// rows of d bf16 each, 16 bytes per lane.  A later destination slot can be
// an earlier row's source (path[t] == t' > t), so every row is read into
// registers before any is written.  Pure data movement, bound by latency:
// one dependent round of loads, then the stores.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxPath = GRAFT_MAX_NODES;  // path entries per request (root included)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(kThreads) void kv_compact_kernel(
    graft_bf16 *__restrict__ kcache, graft_bf16 *__restrict__ vcache, int64_t layer_stride,
    const int64_t *__restrict__ kv_off, int64_t kv_head_stride, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ acc_len,
    const int32_t *__restrict__ acc_path, const int32_t *__restrict__ bonus, int32_t *__restrict__ ctx_next,
    int32_t *__restrict__ root_next, int32_t *__restrict__ err) {
  constexpr int RL = D * 2 / 16;                          // lanes per row (16 bytes each)
  constexpr int PER = 2 * kMaxPath * RL / kThreads;       // (row, piece) pairs per thread
  __shared__ int s_path[kMaxPath];
  __shared__ int s_ok;
  const int h = blockIdx.x, layer = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int ctx = ctx_len[b];
  const int n = n_nodes[b];
  const int a = acc_len[b];
  const int64_t cap = kv_head_stride / D;
  const bool lead = h == 0 && layer == 0;  // writes the request's outputs and flags

  // ---- the path: root first, climbing, inside the tree; the tree inside
  // the cache
  if (tid < 64) {
    const bool len_ok = a >= 0 && a < kMaxPath;
    const int p = (len_ok && tid <= a) ? acc_path[static_cast<size_t>(b) * kMaxPath + tid] : 0;
    const int prev = __shfl(p, tid > 0 ? tid - 1 : 0);
    const bool step_ok = tid > a || (tid == 0 ? p == 0 : (p > prev && p < n));
    const bool path_ok = len_ok && __builtin_amdgcn_ballot_w64(!step_ok) == 0;
    const bool fits = ctx >= 0 && n >= 1 && static_cast<int64_t>(ctx) + n <= cap;
    const bool aligned = (kv_off[b] & 7) == 0;  // rows move 16 bytes at a time
    s_path[tid] = p;
    if (tid == 0) {
      s_ok = path_ok && fits && aligned;
      if (lead && !path_ok) graft::raise_flag(err, GRAFT_ERR_PARENT);
      if (lead && path_ok && !fits) graft::raise_flag(err, GRAFT_ERR_CAPACITY);
      if (lead && !aligned) graft::raise_flag(err, GRAFT_ERR_ALIGN);
    }
  }
  __syncthreads();
  const bool ok = s_ok;
  if (lead && tid == 0) {
    ctx_next[b] = ok ? ctx + a + 1 : ctx;
    root_next[b] = ok ? bonus[b] : -1;
  }
  if (!ok) return;

  // ---- pair q = i * 256 + tid: row m = q / RL (K rows 0..63, V rows
  // 64..127; row t of the path), 16-byte piece q % RL.  Rows with
  // path[t] == t (the root among them) are already in place.
  const int64_t head = kv_off[b] + static_cast<int64_t>(layer) * layer_stride + static_cast<int64_t>(h) * kv_head_stride;
  u32x4 val[PER];
  bool mv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = i * kThreads + tid;
    const int m = q / RL;
    const int t = m & (kMaxPath - 1);
    const int piece = q - m * RL;
    mv[i] = t >= 1 && t <= a && s_path[t] != t;
    if (mv[i]) {
      const graft_bf16 *src = (m < kMaxPath ? kcache : vcache) + head + static_cast<int64_t>(ctx + s_path[t]) * D + piece * 8;
      val[i] = *reinterpret_cast<const u32x4 *>(src);
    }
  }
  // every source row of the workgroup is in registers before any slot is
  // overwritten
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (!mv[i]) continue;
    const int q = i * kThreads + tid;
    const int m = q / RL;
    const int t = m & (kMaxPath - 1);
    const int piece = q - m * RL;
    graft_bf16 *dst = (m < kMaxPath ? kcache : vcache) + head + static_cast<int64_t>(ctx + t) * D + piece * 8;
    *reinterpret_cast<u32x4 *>(dst) = val[i];
  }
}

}  // namespace

extern "C" int graft_kv_compact(int B, int Hkv, int d, int n_layers, graft_bf16 *kcache, graft_bf16 *vcache,
                                int64_t layer_stride, const int64_t *kv_off, int64_t kv_head_stride,
                                const int32_t *ctx_len, const int32_t *n, const int32_t *acc_len,
                                const int32_t *acc_path, const int32_t *bonus, int32_t *ctx_next,
                                int32_t *root_next, int32_t *err_flag, graft_stream stream) {
  using graft::fail;
  if (B < 0 || B > 65535 || Hkv < 1 || Hkv > 65535 || n_layers < 1 || n_layers > 65535)
    return fail(GRAFT_EINVAL, "kv_compact: B=%d Hkv=%d n_layers=%d", B, Hkv, n_layers);
  if (d != 64 && d != 128) return fail(GRAFT_EUNSUPPORTED, "kv_compact: head dim %d (built: 64, 128)", d);
  if (kv_head_stride < d || kv_head_stride % d != 0)
    return fail(GRAFT_EINVAL, "kv_compact: kv_head_stride %lld is not a positive multiple of d",
                static_cast<long long>(kv_head_stride));
  if (n_layers > 1 && layer_stride <= 0)
    return fail(GRAFT_EINVAL, "kv_compact: layer_stride %lld with %d layers", static_cast<long long>(layer_stride),
                n_layers);
  if (B == 0) return GRAFT_OK;
  if (!kcache || !vcache || !kv_off || !ctx_len || !n || !acc_len || !acc_path || !bonus || !ctx_next || !root_next)
    return fail(GRAFT_EINVAL, "kv_compact: NULL array");
  if (ctx_next == ctx_len) return fail(GRAFT_EINVAL, "kv_compact: ctx_next must not alias ctx_len");
  if (!graft::aligned16(kcache) || !graft::aligned16(vcache) || (n_layers > 1 && layer_stride % 8 != 0))
    return fail(GRAFT_EINVAL, "kv_compact: kcache and vcache must be 16-byte aligned, layer_stride a multiple of 8");
  graft::clear_error();
  const dim3 grid(Hkv, n_layers, B);
  if (d == 128)
    hipLaunchKernelGGL((kv_compact_kernel<128>), grid, dim3(kThreads), 0, graft::as_stream(stream), kcache, vcache,
                       layer_stride, kv_off, kv_head_stride, ctx_len, n, acc_len, acc_path, bonus, ctx_next, root_next,
                       err_flag);
  else
    hipLaunchKernelGGL((kv_compact_kernel<64>), grid, dim3(kThreads), 0, graft::as_stream(stream), kcache, vcache,
                       layer_stride, kv_off, kv_head_stride, ctx_len, n, acc_len, acc_path, bonus, ctx_next, root_next,
                       err_flag);
  return graft::check_launch("kv_compact");
}
