// Tree construction, flattening, depth / positions / ancestor mask.
//
// Draft selection: the root plus the best budget-1 candidates by cumulative
// score, a global prune (TreeGraft page, section 3 and section 4 "How";
// Graft page, section 2, second step for the 8/24/40-of-60 stage budgets).
// Retrieved nodes fill the freed slots under the root (Graft page, section
// 2, second step).  The hybrid tree is flattened and gets tree positions
// and a mask (Graft page, section 2, third step).  Static replacement keeps
// the slot count and swaps low-confidence draft nodes for table successors
// (Graft page, section 4, batched-serving paragraph).
//
// One workgroup of 512 threads per request.  Every input array is staged in
// LDS by one round of loads.  Ranking is a rank count: one candidate per
// thread compares its 64-bit key with every other key (broadcast LDS reads,
// one unsigned compare per pair), and a wavefront stops as soon as each of
// its candidates already has budget-1 better ones.  Flattened indices come
// from a ballot / bit-count prefix scan.  The <= 64 flattened nodes map one
// per lane of wave 0, where ancestor masks and depths come from six rounds
// of pointer jumping over the parent links.
#include "common.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWavesBT = kThreads / 64;
constexpr int kPasses = GRAFT_MAX_CAND / kThreads;  // candidate passes of one thread

__device__ void write_padding(int from, int to, int32_t *parent, int32_t *token, int32_t *depth,
                              int32_t *pos, uint64_t *mask, int8_t *src) {
  for (int r = from + static_cast<int>(threadIdx.x); r < to; r += kThreads) {
    parent[r] = -1;
    token[r] = -1;
    depth[r] = -1;
    pos[r] = -1;
    mask[r] = 0;
    src[r] = -1;
  }
}

__global__ __launch_bounds__(kThreads) void build_tree_kernel(
    int mode, const int32_t *__restrict__ cand_parent, const int32_t *__restrict__ cand_token,
    const float *__restrict__ cand_score, const int32_t *__restrict__ cand_off, int max_cand,
    const int32_t *__restrict__ budget, const int32_t *__restrict__ ret_token,
    const int32_t *__restrict__ ret_parent, const int32_t *__restrict__ ret_off,
    const int32_t *__restrict__ table, int V, int k, float thresh,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ row_off,
    int32_t *__restrict__ n_out, int32_t *__restrict__ o_parent, int32_t *__restrict__ o_token,
    int32_t *__restrict__ o_depth, int32_t *__restrict__ o_pos, uint64_t *__restrict__ o_mask,
    int8_t *__restrict__ o_src, int32_t *__restrict__ err) {
  __shared__ float s_score[GRAFT_MAX_CAND];
  __shared__ __attribute__((aligned(16))) uint64_t s_key[GRAFT_MAX_CAND];
  __shared__ int s_par[GRAFT_MAX_CAND];
  __shared__ int s_ctok[GRAFT_MAX_CAND];
  __shared__ int s_idx[GRAFT_MAX_CAND];  // flattened index or -1
  __shared__ int s_wtot[kPasses * kWavesBT];
  __shared__ int s_np[GRAFT_MAX_NODES];
  __shared__ int s_nt[GRAFT_MAX_NODES];
  __shared__ int s_nsrc[GRAFT_MAX_NODES];
  __shared__ int s_low[GRAFT_MAX_NODES];
  __shared__ int s_rpar[GRAFT_MAX_NODES];
  __shared__ int s_rtok[GRAFT_MAX_NODES];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane64 = tid & 63;
  const int c0 = cand_off[b];
  const int C = cand_off[b + 1] - c0;
  const int r0 = row_off[b];
  const int rows = row_off[b + 1] - r0;
  const int cap = rows < GRAFT_MAX_NODES ? rows : GRAFT_MAX_NODES;
  const int R = (mode == GRAFT_TREE_PRUNE && ret_off) ? ret_off[b + 1] - ret_off[b] : 0;
  const int ro = R > 0 ? ret_off[b] : 0;
  const int bud = budget[b];
  const int ctx = ctx_len[b];

  if (C < 1 || C > max_cand || bud < 1 || R < 0) {
    if (tid == 0) {
      graft::raise_flag(err, GRAFT_ERR_CAPACITY);
      n_out[b] = 0;
    }
    write_padding(r0, r0 + rows, o_parent, o_token, o_depth, o_pos, o_mask, o_src);
    return;
  }

  // Stage everything in one round of loads.  Ranking key of candidate c >= 1:
  // (order(score) << 11) | (2047 - c), so "o ranks before c" (higher score,
  // ties to the lower index) is exactly key_o > key_c; the root's slot and
  // the padding hold key 0, below every real key.
  const int Cp = (C + 1) & ~1;
  for (int c = tid; c < Cp; c += kThreads) {
    uint64_t key = 0;
    if (c < C) {
      const float sc = cand_score[c0 + c];
      const int p = cand_parent[c0 + c];
      const int t = cand_token[c0 + c];
      const bool pok = c == 0 ? p == -1 : (p >= 0 && p < c);
      if (!pok) graft::raise_flag(err, GRAFT_ERR_PARENT);
      if (t < 0 || t >= V) graft::raise_flag(err, GRAFT_ERR_TOKEN);
      s_score[c] = sc;
      s_par[c] = p;
      s_ctok[c] = t;
      if (c > 0) key = (static_cast<uint64_t>(graft::float_order(sc)) << 11) | static_cast<uint64_t>(2047 - c);
    }
    s_key[c] = key;
  }
  for (int r = tid; r < R && r < GRAFT_MAX_NODES; r += kThreads) {
    s_rpar[r] = ret_parent[ro + r];
    s_rtok[r] = ret_token[ro + r];
  }
  __syncthreads();

  // keep the root and every candidate with fewer than bud-1 better others;
  // one candidate per thread, one 64-bit compare per (candidate, other) pair
  // on broadcast LDS reads; a wavefront stops once each of its candidates
  // already has bud-1 better ones
  const uint64_t need = static_cast<uint64_t>(bud - 1);
  const ulonglong2 *kv = reinterpret_cast<const ulonglong2 *>(s_key);
  for (int pass = 0; pass < kPasses; ++pass) {
    if (pass * kThreads >= C) break;  // uniform
    const int c = pass * kThreads + tid;
    const bool live = c < C;
    const uint64_t kc = live ? s_key[c] : ~0ull;  // padding lanes count nothing
    uint64_t cnt = 0;
    for (int o2 = 0; o2 < Cp / 2; o2 += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const ulonglong2 q = kv[min(o2 + u, Cp / 2 - 1)];
        const uint64_t w = o2 + u < Cp / 2 ? 1ull : 0ull;
        cnt += (q.x > kc ? w : 0ull) + (q.y > kc ? w : 0ull);
      }
      // every live candidate of this wavefront already excluded (the root
      // stays in regardless)
      if (__builtin_amdgcn_ballot_w64(live && c > 0 && cnt < need) == 0) break;
    }
    const bool keep = live && (c == 0 || cnt < need);
    // exclusive prefix of the keep flags: bit count below this lane within
    // the wavefront, then the totals of the earlier wavefronts
    const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
    if (lane64 == 0) s_wtot[pass * kWavesBT + wave] = __popcll(m);
    if (live) s_idx[c] = keep ? below : -1;
  }
  __syncthreads();
  int nd = 0;
  const int nw = ((C + kThreads - 1) / kThreads) * kWavesBT;
  for (int w2 = 0; w2 < nw; ++w2) nd += s_wtot[w2];
  for (int pass = 0; pass < kPasses; ++pass) {
    const int c = pass * kThreads + tid;
    if (c >= C) break;
    const int i = s_idx[c];
    if (i >= 0) {
      int base = 0;
      for (int w2 = 0; w2 < pass * kWavesBT + wave; ++w2) base += s_wtot[w2];
      s_idx[c] = base + i;
    }
  }
  __syncthreads();

  const int n = nd + R;
  if (n > cap) {
    if (tid == 0) {
      graft::raise_flag(err, GRAFT_ERR_CAPACITY);
      n_out[b] = 0;
    }
    write_padding(r0, r0 + rows, o_parent, o_token, o_depth, o_pos, o_mask, o_src);
    return;
  }

  for (int c = tid; c < C; c += kThreads) {
    int i = s_idx[c];
    if (i < 0) continue;
    int p = -1;
    if (c > 0) {
      int pc = s_par[c];
      p = (pc >= 0 && pc < c) ? s_idx[pc] : -1;
      if (p < 0) {
        graft::raise_flag(err, GRAFT_ERR_NOT_CLOSED);
        p = 0;
      }
    }
    s_np[i] = p;
    s_nt[i] = s_ctok[c];
    s_nsrc[i] = c == 0 ? GRAFT_SRC_ROOT : GRAFT_SRC_DRAFT;
    s_low[i] = (c > 0 && s_score[c] < thresh) ? 1 : 0;
  }
  for (int r = tid; r < R; r += kThreads) {
    int tp = s_rpar[r];
    int p = tp < 0 ? 0 : nd + tp;
    if (tp >= r) {
      graft::raise_flag(err, GRAFT_ERR_PARENT);
      p = 0;
    }
    int t = s_rtok[r];
    if (t < 0 || t >= V) graft::raise_flag(err, GRAFT_ERR_TOKEN);
    s_np[nd + r] = p;
    s_nt[nd + r] = t;
    s_nsrc[nd + r] = GRAFT_SRC_RETRIEVED;
    s_low[nd + r] = 0;
  }
  __syncthreads();

  if (tid < 64) {
    const int lane = tid;
    const bool valid = lane < n;
    const int par = valid ? s_np[lane] : -1;
    int p = par;
    uint64_t m = valid ? (1ull << lane) : 0ull;
    for (int step = 0; step < 6; ++step) {
      const int from = p >= 0 ? p : lane;
      uint64_t mp = __shfl(m, from);
      int pp = __shfl(p, from);
      if (p >= 0) {
        m |= mp;
        p = pp;
      }
    }
    const int dep = valid ? __popcll(m) - 1 : -1;
    int tok = valid ? s_nt[lane] : -1;
    int srcv = valid ? s_nsrc[lane] : -1;

    if (mode == GRAFT_TREE_STATIC_REPLACE) {
      const bool low = valid && s_low[lane];
      int j = 0;
      for (int o = 1; o < lane; ++o) j += (s_low[o] && s_np[o] == par) ? 1 : 0;
      int maxd = dep;
      for (int off = 32; off > 0; off >>= 1) {
        int v = __shfl_xor(maxd, off);
        maxd = v > maxd ? v : maxd;
      }
      for (int level = 1; level <= maxd; ++level) {
        int ptok = __shfl(tok, par >= 0 ? par : lane);
        if (low && dep == level && j < k) {
          if (ptok >= 0 && ptok < V) {
            int t2 = table[static_cast<size_t>(ptok) * k + j];
            if (t2 >= 0 && t2 < V) {
              tok = t2;
              srcv = GRAFT_SRC_REPLACED;
            } else {
              graft::raise_flag(err, GRAFT_ERR_TOKEN);
            }
          } else {
            graft::raise_flag(err, GRAFT_ERR_TOKEN);
          }
        }
      }
    }
    if (valid) {
      const int r = r0 + lane;
      o_parent[r] = par;
      o_token[r] = tok;
      o_depth[r] = dep;
      o_pos[r] = ctx + dep;
      o_mask[r] = m;
      o_src[r] = static_cast<int8_t>(srcv);
    }
    if (lane == 0) n_out[b] = n;
  }
  write_padding(r0 + n, r0 + rows, o_parent, o_token, o_depth, o_pos, o_mask, o_src);
}

}  // namespace

extern "C" int graft_build_tree(int B, int mode, const int32_t *cand_parent, const int32_t *cand_token,
                                const float *cand_score, const int32_t *cand_off, int max_cand,
                                const int32_t *budget, const int32_t *ret_token,
                                const int32_t *ret_parent, const int32_t *ret_off,
                                const int32_t *table, int V, int k, float replace_thresh,
                                const int32_t *ctx_len, const int32_t *row_off, int32_t *n_out,
                                int32_t *parent, int32_t *token, int32_t *depth, int32_t *pos,
                                uint64_t *mask, int8_t *src, int32_t *err_flag, graft_stream stream) {
  using graft::fail;
  if (B < 0) return fail(GRAFT_EINVAL, "build_tree: B=%d", B);
  if (mode != GRAFT_TREE_PRUNE && mode != GRAFT_TREE_STATIC_REPLACE)
    return fail(GRAFT_EINVAL, "build_tree: unknown mode %d", mode);
  if (V <= 0) return fail(GRAFT_EINVAL, "build_tree: V=%d", V);
  if (max_cand < 1 || max_cand > GRAFT_MAX_CAND)
    return fail(GRAFT_EINVAL, "build_tree: max_cand=%d (1..%d)", max_cand, GRAFT_MAX_CAND);
  if (B == 0) return GRAFT_OK;
  if (!cand_parent || !cand_token || !cand_score || !cand_off || !budget || !ctx_len || !row_off ||
      !n_out || !parent || !token || !depth || !pos || !mask || !src)
    return fail(GRAFT_EINVAL, "build_tree: NULL array");
  if (mode == GRAFT_TREE_PRUNE && ret_off && (!ret_token || !ret_parent))
    return fail(GRAFT_EINVAL, "build_tree: ret_off given without ret_token/ret_parent");
  if (mode == GRAFT_TREE_STATIC_REPLACE && (!table || k < 1 || k > GRAFT_MAX_K))
    return fail(GRAFT_EINVAL, "build_tree: static replacement needs table and 1<=k<=%d", GRAFT_MAX_K);
  graft::clear_error();
  hipLaunchKernelGGL(build_tree_kernel, dim3(B), dim3(kThreads), 0, graft::as_stream(stream), mode,
                     cand_parent, cand_token, cand_score, cand_off, max_cand, budget, ret_token,
                     ret_parent, ret_off, table, V, k, replace_thresh, ctx_len, row_off, n_out, parent,
                     token, depth, pos, mask, src, err_flag);
  return graft::check_launch("build_tree");
}
