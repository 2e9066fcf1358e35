// Greedy acceptance on the verified tree.
//
// Graft page (arXiv:2605.20104 write-up), section 2, third step: draft and
// retrieved nodes face the same verification rule.  At temperature 0
// (TreeGraft page, section 5) a node is accepted when its token equals the
// target's argmax at its parent and the parent is accepted; the round keeps
// the deepest accepted root path (TreeGraft page, section 1: acceptance
// stops at the first rejection).
//
// One wavefront per request, one lane per node (trees have <= 64 nodes).
// "accepted" is the AND of the edge tests along the root path and depth is
// the path length: both come from six rounds of pointer jumping, the
// deepest accepted node from a wave max-reduction of (depth, -index), and
// the path from that node's ancestor bitmask.
//
// Sampling at temperature T > 0 (FIRST_MATCH): "argmax" is the token drawn at
// each node, and only the lowest-index child matching its parent's draw is
// accepted, so the accepted set is one chain and every emitted token follows
// the target's distribution (rejection sampling keeps it unchanged: TreeGraft
// page, section 3 and its reading list; the rule for several children is
// this library's reading, the pages give none).
#include "common.h"

namespace {

template <bool FIRST_MATCH>
__global__ __launch_bounds__(64) void accept_kernel(const int32_t *__restrict__ n_arr,
                                                    const int32_t *__restrict__ row_off,
                                                    const int32_t *__restrict__ parent,
                                                    const int32_t *__restrict__ token,
                                                    const int32_t *__restrict__ topk_id, int k,
                                                    int32_t *__restrict__ acc_len,
                                                    int32_t *__restrict__ acc_path,
                                                    int32_t *__restrict__ bonus,
                                                    int32_t *__restrict__ err) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  // Two rounds of loads in all: the request's scalars, then every node array
  // (their addresses depend only on row_off[b]).  Each round is used once
  // before anything else, so no test or branch splits it into a chain.
  const int r0 = row_off[b];
  const int r1 = row_off[b + 1];
  const int n = n_arr[b];
  asm volatile("" ::"s"(r0), "s"(r1), "s"(n), "s"(parent), "s"(token), "s"(topk_id), "s"(k));  // and the arguments
  __builtin_amdgcn_sched_barrier(0);
  const int cap = r1 - r0;
  // lanes within the request's row capacity read its rows (padding rows
  // included: they belong to the request); the rest read nothing
  const bool in_cap = lane < cap;
  const int par_ld = in_cap ? parent[r0 + lane] : -1;
  const int tok_ld = in_cap ? token[r0 + lane] : -1;
  const int am_ld = in_cap ? topk_id[static_cast<size_t>(r0 + lane) * k] : -1;
  asm volatile("" ::"v"(par_ld), "v"(tok_ld), "v"(am_ld));
  __builtin_amdgcn_sched_barrier(0);
  int32_t *path = acc_path + static_cast<size_t>(b) * GRAFT_MAX_NODES;

  if (n < 1 || n > cap || n > GRAFT_MAX_NODES) {
    if (lane == 0) {
      graft::raise_flag(err, GRAFT_ERR_CAPACITY);
      acc_len[b] = 0;
      bonus[b] = (n >= 1 && cap >= 1) ? topk_id[static_cast<size_t>(r0) * k] : -1;
    }
    path[lane] = lane == 0 ? 0 : -1;
    return;
  }

  const bool valid = lane < n;
  const int par = valid ? par_ld : -1;
  const bool pok = !valid || (lane == 0 ? par == -1 : (par >= 0 && par < lane));
  const unsigned long long badmask = __ballot(!pok);
  if (badmask) {
    if (lane == 0) {
      graft::raise_flag(err, GRAFT_ERR_PARENT);
      acc_len[b] = 0;
      bonus[b] = topk_id[static_cast<size_t>(r0) * k];
    }
    path[lane] = lane == 0 ? 0 : -1;
    return;
  }

  const int am = valid ? am_ld : -1;  // argmax of this node
  const int tok = valid ? tok_ld : -1;
  // edge test: my token against my parent's argmax
  const int parent_am = __shfl(am, par >= 0 ? par : lane);
  int ok = (lane == 0) ? 1 : (valid && tok == parent_am ? 1 : 0);
  if constexpr (FIRST_MATCH) {
    // an earlier sibling that matches the same draw takes it
    const int mk = (ok && lane > 0) ? par : -2;
    int earlier = 0;
    for (int o = 1; o < n; ++o) {
      const int v = __builtin_amdgcn_readlane(mk, o);
      earlier |= (o < lane && v == par) ? 1 : 0;
    }
    if (earlier) ok = 0;
  }
  int dep = (valid && lane > 0) ? 1 : 0;
  uint64_t anc = valid ? (1ull << lane) : 0ull;
  int p = par;
  for (int step = 0; step < 6; ++step) {
    const int from = p >= 0 ? p : lane;
    const int ok_p = __shfl(ok, from);
    const int dep_p = __shfl(dep, from);
    const uint64_t anc_p = __shfl(anc, from);
    const int p_p = __shfl(p, from);
    if (p >= 0) {
      ok &= ok_p;
      dep += dep_p;
      anc |= anc_p;
      p = p_p;
    }
  }
  // deepest accepted node, ties to the lowest index
  int key = (valid && ok) ? (dep << 6) | (63 - lane) : -1;
  for (int off = 32; off > 0; off >>= 1) {
    int o = __shfl_xor(key, off);
    key = o > key ? o : key;
  }
  const int best = 63 - (key & 63);
  const int a = key >> 6;
  const uint64_t best_anc = __shfl(anc, best);
  const int best_am = __shfl(am, best);

  if ((best_anc >> lane) & 1ull) path[dep] = lane;  // on best's root path: slot = depth
  if (lane > a) path[lane] = -1;
  if (lane == 0) {
    acc_len[b] = a;
    bonus[b] = best_am;
  }
}

}  // namespace

extern "C" int graft_accept(int B, const int32_t *n, const int32_t *row_off, const int32_t *parent,
                            const int32_t *token, const int32_t *topk_id, int k, int32_t *acc_len,
                            int32_t *acc_path, int32_t *bonus, int32_t *err_flag, graft_stream stream) {
  using graft::fail;
  if (B < 0 || k < 1 || k > GRAFT_MAX_K) return fail(GRAFT_EINVAL, "accept: B=%d k=%d", B, k);
  if (B == 0) return GRAFT_OK;
  if (!n || !row_off || !parent || !token || !topk_id || !acc_len || !acc_path || !bonus)
    return fail(GRAFT_EINVAL, "accept: NULL array");
  graft::clear_error();
  hipLaunchKernelGGL(accept_kernel<false>, dim3(B), dim3(64), 0, graft::as_stream(stream), n, row_off, parent,
                     token, topk_id, k, acc_len, acc_path, bonus, err_flag);
  return graft::check_launch("accept");
}

extern "C" int graft_accept_sampled(int B, const int32_t *n, const int32_t *row_off, const int32_t *parent,
                                    const int32_t *token, const int32_t *sample_id, int32_t *acc_len,
                                    int32_t *acc_path, int32_t *bonus, int32_t *err_flag, graft_stream stream) {
  using graft::fail;
  if (B < 0) return fail(GRAFT_EINVAL, "accept_sampled: B=%d", B);
  if (B == 0) return GRAFT_OK;
  if (!n || !row_off || !parent || !token || !sample_id || !acc_len || !acc_path || !bonus)
    return fail(GRAFT_EINVAL, "accept_sampled: NULL array");
  graft::clear_error();
  hipLaunchKernelGGL(accept_kernel<true>, dim3(B), dim3(64), 0, graft::as_stream(stream), n, row_off, parent,
                     token, sample_id, 1, acc_len, acc_path, bonus, err_flag);
  return graft::check_launch("accept_sampled");
}
