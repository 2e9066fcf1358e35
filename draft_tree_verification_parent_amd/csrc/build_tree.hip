// Tree construction, flattening, depth / positions / ancestor mask.
//
// Draft selection: the root plus the best budget-1 candidates by cumulative
// score, a global prune (TreeGraft page, section 3 and section 4 "How";
// Graft page, section 2, second step for the 8/24/40-of-60 stage budgets).
// Retrieved nodes fill the freed slots under the root (Graft page, section
// 2, second step).  The hybrid tree is flattened and gets tree positions
// and a mask (Graft page, section 2, third step).  Static replacement keeps
// the slot count and swaps low-confidence draft nodes for table successors
// (Graft page, section 4, batched-serving paragraph).  Tail mode (Graft page,
// section 7, Graft-TAIL on block drafts): the candidates are a block draft
// with per-token confidences; the prefix up to the first confidence below
// tau is kept and the freed slots take the first template rows, hung under
// the deepest kept node.
//
// One workgroup of 512 threads per request.  Every input array is staged in
// LDS by one round of loads.  Ranking works on unique 64-bit keys: each
// wavefront sorts its blocks of 64 keys in registers (bitonic network over
// DPP and row-swap permutes) and keeps the 64 largest; pairwise bitonic
// merges across wavefronts give the request's 64 largest keys, and with
// them the smallest key within the budget, against which every candidate
// is tested.  Flattened indices come from a ballot / bit-count prefix scan.
// The <= 64 flattened nodes map one per lane of wave 0, where ancestor masks
// and depths come from six rounds of pointer jumping over the parent links;
// static replacement looks up the table in rounds, one per link of the
// longest chain of replaced nodes.
#include "common.h"
#include "topk_list.h"

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

using graft::lane_xor32;

template <int J>
__device__ inline uint64_t lane_xor(uint64_t x, int lane) {
  const uint32_t lo = lane_xor32<J>(static_cast<uint32_t>(x), lane);
  const uint32_t hi = lane_xor32<J>(static_cast<uint32_t>(x >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One compare-exchange stage of a bitonic network over the 64 lanes: pairs
// (i, i ^ J); within K-blocks whose index bit K is clear the lower lane keeps
// the larger key (the smaller when the whole network sorts ascending).
template <int K, int J>
__device__ inline uint64_t bitonic_step(uint64_t x, int lane, bool desc) {
  const uint64_t y = lane_xor<J>(x, lane);
  const bool keep_max = (((lane & K) == 0) == ((lane & J) == 0)) == desc;
  return keep_max ? (x > y ? x : y) : (x < y ? x : y);
}

// Sorts the 64 keys of a wavefront, largest in lane 0 when desc, smallest
// otherwise.
__device__ inline uint64_t wave_sort(uint64_t x, int lane, bool desc) {
  x = bitonic_step<2, 1>(x, lane, desc);
  x = bitonic_step<4, 2>(x, lane, desc);
  x = bitonic_step<4, 1>(x, lane, desc);
  x = bitonic_step<8, 4>(x, lane, desc);
  x = bitonic_step<8, 2>(x, lane, desc);
  x = bitonic_step<8, 1>(x, lane, desc);
  x = bitonic_step<16, 8>(x, lane, desc);
  x = bitonic_step<16, 4>(x, lane, desc);
  x = bitonic_step<16, 2>(x, lane, desc);
  x = bitonic_step<16, 1>(x, lane, desc);
  x = bitonic_step<32, 16>(x, lane, desc);
  x = bitonic_step<32, 8>(x, lane, desc);
  x = bitonic_step<32, 4>(x, lane, desc);
  x = bitonic_step<32, 2>(x, lane, desc);
  x = bitonic_step<32, 1>(x, lane, desc);
  x = bitonic_step<64, 32>(x, lane, desc);
  x = bitonic_step<64, 16>(x, lane, desc);
  x = bitonic_step<64, 8>(x, lane, desc);
  x = bitonic_step<64, 4>(x, lane, desc);
  x = bitonic_step<64, 2>(x, lane, desc);
  return bitonic_step<64, 1>(x, lane, desc);
}

// Top 64 of two sorted blocks, a in direction desc and b in the opposite
// one: their lane-wise maximum is a bitonic sequence holding the 64 largest
// keys of both, which the last six stages of the network then sort.
__device__ inline uint64_t top64_merge(uint64_t a, uint64_t b, int lane, bool desc) {
  uint64_t x = a > b ? a : b;
  x = bitonic_step<64, 32>(x, lane, desc);
  x = bitonic_step<64, 16>(x, lane, desc);
  x = bitonic_step<64, 8>(x, lane, desc);
  x = bitonic_step<64, 4>(x, lane, desc);
  x = bitonic_step<64, 2>(x, lane, desc);
  return bitonic_step<64, 1>(x, lane, desc);
}

// The 64 largest keys of a 512-thread workgroup (thread tid holds the key of
// item p * 512 + tid in kreg[p]; NB = number of 64-item blocks in use),
// sorted descending, in the lanes of wavefront 0 (other wavefronts: partial
// results).  Each wavefront sorts its blocks in registers and keeps the top
// 64; three rounds of pairwise merges through LDS follow, partners sorted in
// opposite directions.  Every thread must call it (three barriers).
__device__ inline uint64_t workgroup_top64(const uint64_t (&kreg)[kPasses], int NB, int wave, int lane,
                                           uint64_t (*s_m1)[64], uint64_t (*s_m2)[64], uint64_t *s_m3) {
  const bool dir0 = (wave & 1) == 0;
  uint64_t top = wave_sort(kreg[0], lane, dir0);
#pragma unroll
  for (int pass = 1; pass < kPasses; ++pass)
    if (pass * kWavesBT < NB)  // uniform
      top = top64_merge(top, wave_sort(kreg[pass], lane, !dir0), lane, dir0);
  if (wave & 1) s_m1[wave >> 1][lane] = top;
  __syncthreads();
  if (!(wave & 1)) top = top64_merge(top, s_m1[wave >> 1][lane], lane, ((wave >> 1) & 1) == 0);
  if ((wave & 3) == 2) s_m2[wave >> 2][lane] = top;
  __syncthreads();
  if ((wave & 3) == 0) top = top64_merge(top, s_m2[wave >> 2][lane], lane, ((wave >> 2) & 1) == 0);
  if (wave == 4) s_m3[lane] = top;
  __syncthreads();
  if (wave == 0) top = top64_merge(top, s_m3[lane], lane, true);
  return top;
}

__global__ __launch_bounds__(kThreads) void build_tree_kernel(
    int mode, const int32_t *__restrict__ cand_parent, const int32_t *__restrict__ cand_token,
    const float *__restrict__ cand_score, const int32_t *__restrict__ cand_off, int max_cand,
    const int32_t *__restrict__ budget, const int32_t *__restrict__ ret_token,
    const int32_t *__restrict__ ret_parent, const int32_t *__restrict__ ret_off,
    const int32_t *__restrict__ ret_anchor, const int32_t *__restrict__ table, int V, int k, float thresh,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ row_off,
    int32_t *__restrict__ n_out, int32_t *__restrict__ o_parent, int32_t *__restrict__ o_token,
    int32_t *__restrict__ o_depth, int32_t *__restrict__ o_pos, uint64_t *__restrict__ o_mask,
    int8_t *__restrict__ o_src, int32_t *__restrict__ err) {
  __shared__ float s_score[GRAFT_MAX_CAND];
  __shared__ int s_par[GRAFT_MAX_CAND];
  __shared__ int s_ctok[GRAFT_MAX_CAND];
  __shared__ int s_idx[GRAFT_MAX_CAND];  // flattened index or -1
  __shared__ int s_wtot[kPasses * kWavesBT];
  __shared__ uint64_t s_m1[4][64], s_m2[2][64], s_m3[64];  // merge partners, one buffer per round
  __shared__ uint64_t s_thr;                                // smallest key kept
  __shared__ int s_firstlow;                                // tail mode: first block index below tau
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
  const bool tail = mode == GRAFT_TREE_TAIL;
  const int R = ((mode == GRAFT_TREE_PRUNE || tail) && ret_off) ? ret_off[b + 1] - ret_off[b] : 0;
  const int ro = R > 0 ? ret_off[b] : 0;
  const int bud = budget[b];
  const int ctx = ctx_len[b];
  // candidate under which retrieved nodes with template parent -1 hang
  const int anc_c = (mode == GRAFT_TREE_PRUNE && ret_anchor) ? ret_anchor[b] : 0;

  if (C < 1 || C > max_cand || bud < 1 || R < 0) {
    if (tid == 0) {
      graft::raise_flag(err, GRAFT_ERR_CAPACITY);
      n_out[b] = 0;
    }
    write_padding(r0, r0 + rows, o_parent, o_token, o_depth, o_pos, o_mask, o_src);
    return;
  }

  // Stage everything in one round of loads.  Ranking key of candidate c >= 1:
  // 2^43 | (order(score) << 11) | (2047 - c), so "o ranks before c" (higher
  // score, ties to the lower index) is exactly key_o > key_c; the root and
  // the padding hold key 0, below every real key.  Thread tid holds the key
  // of candidate p * 512 + tid, so wavefront w of pass p holds block 8p + w.
  uint64_t kreg[kPasses];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int c = pass * kThreads + tid;
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
      if (c > 0)
        key = (1ull << 43) | (static_cast<uint64_t>(graft::float_order(sc)) << 11) |
              static_cast<uint64_t>(2047 - c);
    }
    kreg[pass] = key;
  }
  if (tid == 0) s_firstlow = C;
  for (int r = tid; r < R && r < GRAFT_MAX_NODES; r += kThreads) {
    s_rpar[r] = ret_parent[ro + r];
    s_rtok[r] = ret_token[ro + r];
  }
  // Keep the root and the bud-1 best other candidates.  Each wavefront sorts
  // its 64-key blocks in registers and folds them into the sorted 64 largest
  // of its keys; three rounds of pairwise merges across wavefronts leave the
  // 64 largest keys of the request in wavefront 0, where entry bud-2 is the
  // smallest key kept.  Merge partners are sorted in opposite directions.
  const uint64_t top = workgroup_top64(kreg, (C + 63) / 64, wave, lane64, s_m1, s_m2, s_m3);
  const int need = bud - 1;
  if (wave == 0) {
    // need > 64 keeps the 64 largest, already more than a request can hold
    const int at = need <= 0 ? 0 : (need < 64 ? need - 1 : 63);
    if (lane64 == at) s_thr = need <= 0 ? ~0ull : top;
  }
  // tail mode: candidates 0..K are kept, K + 1 = the first block index whose
  // confidence is below tau (NaN counts as below)
  if (tail) {
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int c = pass * kThreads + tid;
      if (c >= 1 && c < C && !(s_score[c] >= thresh)) atomicMin(&s_firstlow, c);
    }
  }
  __syncthreads();
  const uint64_t thr = s_thr;
  const int firstlow = s_firstlow;
  // exclusive prefix of the keep flags: bit count below this lane within the
  // wavefront, then the totals of the earlier wavefronts
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    if (pass * kThreads < C) {  // uniform
      const int c = pass * kThreads + tid;
      const bool live = c < C;
      const bool keep = live && (tail ? c < firstlow : (c == 0 || kreg[pass] >= thr));
      const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
      const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
      if (lane64 == 0) s_wtot[pass * kWavesBT + wave] = __popcll(m);
      if (live) s_idx[c] = keep ? below : -1;
    }
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

  // tail mode: the retrieved rows fill the budget left after the kept prefix
  // (the template's first rows are the smaller templates)
  const int Rk = tail ? max(0, min(R, bud - nd)) : R;
  const int n = nd + Rk;
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
  // the anchor must be a kept candidate (the root always is)
  int anc_i = 0;
  if (anc_c != 0) {
    anc_i = (anc_c > 0 && anc_c < C) ? s_idx[anc_c] : -1;
    if (anc_i < 0) {
      if (tid == 0) graft::raise_flag(err, GRAFT_ERR_NOT_CLOSED);
      anc_i = 0;
    }
  }
  for (int r = tid; r < Rk; r += kThreads) {
    int tp = s_rpar[r];
    int p = tp < 0 ? (tail ? nd - 1 : anc_i) : nd + tp;  // tail: under the deepest kept node
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
      // j = index of this node among the low-confidence children of its
      // parent, counted in flattened order
      const int lowpar = (valid && s_low[lane]) ? par : -2;
      int j = 0;
      for (int o = 1; o < n; ++o) {
        const int v = __builtin_amdgcn_readlane(lowpar, o);
        j += (o < lane && v == par) ? 1 : 0;
      }
      // A node is replaced once its parent's token is final; only chains of
      // replaced nodes need further rounds.  Parents precede children, so the
      // first pending node is always ready and the loop ends.
      bool pending = lowpar >= 0 && j < k;
      for (int round = 0; round < GRAFT_MAX_NODES; ++round) {
        if (__builtin_amdgcn_ballot_w64(pending) == 0) break;
        const int from = par >= 0 ? par : lane;
        const int ptok = __shfl(tok, from);
        const bool ppend = __shfl(static_cast<int>(pending), from) != 0;
        if (pending && !ppend) {
          if (ptok >= 0 && ptok < V) {
            const int t2 = table[static_cast<size_t>(ptok) * k + j];
            if (t2 >= 0 && t2 < V) {
              tok = t2;
              srcv = GRAFT_SRC_REPLACED;
            } else {
              graft::raise_flag(err, GRAFT_ERR_TOKEN);
            }
          } else {
            graft::raise_flag(err, GRAFT_ERR_TOKEN);
          }
          pending = false;
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

// Nodes TreeGraft's construction creates (root included): sizes and the
// schedule decide it, not the data.  -1 if a step would exceed max_nodes.
__host__ __device__ inline int treegraft_count(int D, int W, int m, int mid_mask, int max_nodes) {
  int n = 1, newest = 1, visited = 0;
  for (int k = 0; k < D; ++k) {
    const bool mid = (mid_mask >> k) & 1;
    const int pool = mid ? n - visited : newest;
    const int f = pool < W ? pool : W;
    if (mid) visited = n;
    newest = f * m;
    n += newest;
    if (n > max_nodes) return -1;
  }
  return n;
}

// Retrieval anchor of a tree pruned at checkpoint depth c (Graft page,
// section 2, second step: the retrieval tree grows from the token generated
// up to the checkpoint).  The current best path at depth c ends at the best
// candidate of that depth (c capped at the deepest candidate depth); the
// anchor is that candidate if the budget keeps it, else its deepest kept
// ancestor.  One 512-thread workgroup per request: the kept threshold comes
// from the same workgroup top-64 as the tree build, candidate depths from
// eleven rounds of pointer jumping in LDS (chains of up to 2048 nodes), the
// best candidate of depth c from an LDS maximum of the unique keys, and one
// thread walks up its path to the first kept node (kept keys are exactly
// those >= the threshold, and a kept node's ancestors are kept).
__global__ __launch_bounds__(kThreads) void prune_anchor_kernel(
    const int32_t *__restrict__ cand_parent, const int32_t *__restrict__ cand_token,
    const float *__restrict__ cand_score, const int32_t *__restrict__ cand_off, int max_cand,
    const int32_t *__restrict__ budget, const int32_t *__restrict__ stage, int32_t *__restrict__ anchor,
    int32_t *__restrict__ anchor_token, int32_t *__restrict__ err) {
  __shared__ int s_par[GRAFT_MAX_CAND];
  __shared__ float s_sc[GRAFT_MAX_CAND];
  __shared__ int s_anc[2][GRAFT_MAX_CAND];
  __shared__ int s_dep[2][GRAFT_MAX_CAND];
  __shared__ uint64_t s_m1[4][64], s_m2[2][64], s_m3[64];
  __shared__ uint64_t s_thr, s_best;
  __shared__ int s_maxdep;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane64 = tid & 63;
  const int c0 = cand_off[b];
  const int C = cand_off[b + 1] - c0;
  const int bud = budget[b];
  const int depth_c = stage[b];
  if (C < 1 || C > max_cand || bud < 1) {
    if (tid == 0) {
      graft::raise_flag(err, GRAFT_ERR_CAPACITY);
      anchor[b] = 0;
      anchor_token[b] = C >= 1 ? cand_token[c0] : -1;
    }
    return;
  }
  uint64_t kreg[kPasses];
  bool bad = false;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int c = pass * kThreads + tid;
    uint64_t key = 0;
    if (c < C) {
      const float sc = cand_score[c0 + c];
      const int p = cand_parent[c0 + c];
      const bool pok = c == 0 ? p == -1 : (p >= 0 && p < c);
      bad |= !pok;
      s_sc[c] = sc;
      s_par[c] = pok ? p : (c == 0 ? -1 : 0);  // a broken link is read as the root's
      s_anc[0][c] = c == 0 ? -1 : s_par[c];
      s_dep[0][c] = c == 0 ? 0 : 1;
      if (c > 0)
        key = (1ull << 43) | (static_cast<uint64_t>(graft::float_order(sc)) << 11) |
              static_cast<uint64_t>(2047 - c);
    }
    kreg[pass] = key;
  }
  if (bad) graft::raise_flag(err, GRAFT_ERR_PARENT);
  if (tid == 0) {
    s_maxdep = 0;
    s_best = 0;
  }
  const uint64_t top = workgroup_top64(kreg, (C + 63) / 64, wave, lane64, s_m1, s_m2, s_m3);
  const int need = bud - 1;
  if (wave == 0) {
    const int at = need <= 0 ? 0 : (need < 64 ? need - 1 : 63);
    if (lane64 == at) s_thr = need <= 0 ? ~0ull : top;
  }
  // depths: after round j, anc is the 2^j-th ancestor (or -1) and dep the
  // distance to it (to the root once anc is -1)
  int cur = 0;
  for (int round = 0; round < 11; ++round) {
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int c = pass * kThreads + tid;
      if (c < C) {
        const int a = s_anc[cur][c];
        s_anc[cur ^ 1][c] = a >= 0 ? s_anc[cur][a] : -1;
        s_dep[cur ^ 1][c] = s_dep[cur][c] + (a >= 0 ? s_dep[cur][a] : 0);
      }
    }
    cur ^= 1;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int c = pass * kThreads + tid;
    if (c < C) atomicMax(&s_maxdep, s_dep[cur][c]);
  }
  __syncthreads();
  const int c_eff = depth_c < s_maxdep ? depth_c : s_maxdep;
  if (c_eff > 0) {
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int c = pass * kThreads + tid;
      if (c >= 1 && c < C && s_dep[cur][c] == c_eff) atomicMax(reinterpret_cast<unsigned long long *>(&s_best),
                                                               static_cast<unsigned long long>(kreg[pass]));
    }
  }
  __syncthreads();
  if (tid == 0) {
    int v = 0;
    if (c_eff > 0 && s_best != 0) {
      const uint64_t thr = s_thr;
      v = 2047 - static_cast<int>(s_best & 2047);
      // climb to the first kept node: key >= thr (the root is always kept)
      while (v != 0) {
        const uint64_t key = (1ull << 43) | (static_cast<uint64_t>(graft::float_order(s_sc[v])) << 11) |
                             static_cast<uint64_t>(2047 - v);
        if (key >= thr) break;
        v = s_par[v];
      }
    }
    anchor[b] = v;
    anchor_token[b] = cand_token[c0 + v];
  }
}

// TreeGraft's shared tree (TreeGraft page, section 3: frontier = best W of
// the pool by cumulative score, m children each; section 4 "Where"/"How": a
// mid-drafter step's pool is every node it has not visited, ranked by its own
// path score; children are appended, never overwriting).  One 512-thread
// workgroup per request; per step the pool's keys (score order << 11 |
// 2047 - node) go through the workgroup top-64, wavefront 0 writes the W
// best to LDS, then every child is created by one thread.  Stored score s and
// mid score r are fp32 products, as the oracle forms them.
__global__ __launch_bounds__(kThreads) void treegraft_kernel(int D, int W, int m, const int32_t *__restrict__ mid_mask,
                                                             const int32_t *__restrict__ root_token,
                                                             const int32_t *__restrict__ tok,
                                                             const float *__restrict__ prob,
                                                             const float *__restrict__ q,
                                                             const int32_t *__restrict__ cand_off,
                                                             int32_t *__restrict__ out_parent,
                                                             int32_t *__restrict__ out_token,
                                                             float *__restrict__ out_score, int32_t *__restrict__ err) {
  __shared__ float s_s[GRAFT_MAX_CAND];
  __shared__ float s_r[GRAFT_MAX_CAND];
  __shared__ signed char s_created[GRAFT_MAX_CAND];
  __shared__ signed char s_visited[GRAFT_MAX_CAND];
  __shared__ uint64_t s_m1[4][64], s_m2[2][64], s_m3[64];
  __shared__ int s_front[64];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int mask = mid_mask[b];
  const int base = cand_off[b];
  const int cap = cand_off[b + 1] - base;
  const int total = treegraft_count(D, W, m, mask, GRAFT_MAX_CAND);
  if (total < 0 || total != cap) {
    if (tid == 0) graft::raise_flag(err, GRAFT_ERR_CAPACITY);
    return;
  }
  const size_t step_stride = static_cast<size_t>(W) * m;
  const int32_t *tok_b = tok + static_cast<size_t>(b) * D * step_stride;
  const float *prob_b = prob + static_cast<size_t>(b) * D * step_stride;
  if (tid == 0) {
    s_s[0] = 1.f;
    s_r[0] = 1.f;
    s_created[0] = 0;
    s_visited[0] = 0;
    out_parent[base] = -1;
    out_token[base] = root_token[b];
    out_score[base] = 1.f;
  }
  __syncthreads();
  int n = 1, newest = 1, visited = 0;
  for (int k = 0; k < D; ++k) {
    const bool mid = (mask >> k) & 1;
    const int pool = mid ? n - visited : newest;
    const int F = pool < W ? pool : W;
    uint64_t kreg[kPasses];
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int v = pass * kThreads + tid;
      uint64_t key = 0;
      if (v < n) {
        const bool in_pool = mid ? !s_visited[v] : s_created[v] == k;
        if (in_pool)
          key = (1ull << 43) | (static_cast<uint64_t>(graft::float_order(mid ? s_r[v] : s_s[v])) << 11) |
                static_cast<uint64_t>(2047 - v);
      }
      kreg[pass] = key;
    }
    const uint64_t top = workgroup_top64(kreg, (n + 63) / 64, wave, lane, s_m1, s_m2, s_m3);
    if (wave == 0 && lane < F) s_front[lane] = 2047 - static_cast<int>(top & 2047);
    if (mid) {
#pragma unroll
      for (int pass = 0; pass < kPasses; ++pass)
        if (kreg[pass] != 0) s_visited[pass * kThreads + tid] = 1;  // the pool is visited now
    }
    __syncthreads();
    for (int t = tid; t < F * m; t += kThreads) {
      const int j = t / m, c = t - j * m;
      const int f = s_front[j];
      const int v = n + t;
      const size_t o = static_cast<size_t>(k) * step_stride + static_cast<size_t>(j) * m + c;
      const float sv = s_s[f] * prob_b[o];
      const float rv = s_r[f] * q[base + v];
      s_s[v] = sv;
      s_r[v] = rv;
      s_created[v] = static_cast<signed char>(k + 1);
      s_visited[v] = 0;
      out_parent[base + v] = f;
      out_token[base + v] = tok_b[o];
      out_score[base + v] = sv;
    }
    __syncthreads();
    if (mid) visited = n;
    newest = F * m;
    n += newest;
  }
}

// Graft-TAIL cut: per request, the number of leading block tokens with
// confidence >= tau (NaN counts as below) and the token at the deepest kept
// node, the retrieval root (the tree root when none is kept).
__global__ __launch_bounds__(256) void tail_cut_kernel(int B, int L, const int32_t *__restrict__ root_token,
                                                       const int32_t *__restrict__ block_token,
                                                       const float *__restrict__ block_conf, float tau,
                                                       int32_t *__restrict__ keep_len,
                                                       int32_t *__restrict__ retrieval_root) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const float *conf = block_conf + static_cast<size_t>(b) * L;
  int K = L;
  for (int i = 0; i < L; ++i)
    if (!(conf[i] >= tau)) {
      K = i;
      break;
    }
  keep_len[b] = K;
  retrieval_root[b] = K == 0 ? root_token[b] : block_token[static_cast<size_t>(b) * L + K - 1];
}

}  // namespace

extern "C" int graft_build_tree(int B, int mode, const int32_t *cand_parent, const int32_t *cand_token,
                                const float *cand_score, const int32_t *cand_off, int max_cand,
                                const int32_t *budget, const int32_t *ret_token,
                                const int32_t *ret_parent, const int32_t *ret_off, const int32_t *ret_anchor,
                                const int32_t *table, int V, int k, float replace_thresh,
                                const int32_t *ctx_len, const int32_t *row_off, int32_t *n_out,
                                int32_t *parent, int32_t *token, int32_t *depth, int32_t *pos,
                                uint64_t *mask, int8_t *src, int32_t *err_flag, graft_stream stream) {
  using graft::fail;
  if (B < 0) return fail(GRAFT_EINVAL, "build_tree: B=%d", B);
  if (mode != GRAFT_TREE_PRUNE && mode != GRAFT_TREE_STATIC_REPLACE && mode != GRAFT_TREE_TAIL)
    return fail(GRAFT_EINVAL, "build_tree: unknown mode %d", mode);
  if (V <= 0) return fail(GRAFT_EINVAL, "build_tree: V=%d", V);
  if (max_cand < 1 || max_cand > GRAFT_MAX_CAND)
    return fail(GRAFT_EINVAL, "build_tree: max_cand=%d (1..%d)", max_cand, GRAFT_MAX_CAND);
  if (B == 0) return GRAFT_OK;
  if (!cand_parent || !cand_token || !cand_score || !cand_off || !budget || !ctx_len || !row_off ||
      !n_out || !parent || !token || !depth || !pos || !mask || !src)
    return fail(GRAFT_EINVAL, "build_tree: NULL array");
  if ((mode == GRAFT_TREE_PRUNE || mode == GRAFT_TREE_TAIL) && ret_off && (!ret_token || !ret_parent))
    return fail(GRAFT_EINVAL, "build_tree: ret_off given without ret_token/ret_parent");
  if (mode == GRAFT_TREE_STATIC_REPLACE && (!table || k < 1 || k > GRAFT_MAX_K))
    return fail(GRAFT_EINVAL, "build_tree: static replacement needs table and 1<=k<=%d", GRAFT_MAX_K);
  graft::clear_error();
  hipLaunchKernelGGL(build_tree_kernel, dim3(B), dim3(kThreads), 0, graft::as_stream(stream), mode,
                     cand_parent, cand_token, cand_score, cand_off, max_cand, budget, ret_token,
                     ret_parent, ret_off, ret_anchor, table, V, k, replace_thresh, ctx_len, row_off, n_out, parent,
                     token, depth, pos, mask, src, err_flag);
  return graft::check_launch("build_tree");
}

extern "C" int graft_prune_anchor(int B, const int32_t *cand_parent, const int32_t *cand_token,
                                  const float *cand_score, const int32_t *cand_off, int max_cand,
                                  const int32_t *budget, const int32_t *stage, int32_t *anchor,
                                  int32_t *anchor_token, int32_t *err_flag, graft_stream stream) {
  using graft::fail;
  if (B < 0) return fail(GRAFT_EINVAL, "prune_anchor: B=%d", B);
  if (max_cand < 1 || max_cand > GRAFT_MAX_CAND)
    return fail(GRAFT_EINVAL, "prune_anchor: max_cand=%d (1..%d)", max_cand, GRAFT_MAX_CAND);
  if (B == 0) return GRAFT_OK;
  if (!cand_parent || !cand_token || !cand_score || !cand_off || !budget || !stage || !anchor || !anchor_token)
    return fail(GRAFT_EINVAL, "prune_anchor: NULL array");
  graft::clear_error();
  hipLaunchKernelGGL(prune_anchor_kernel, dim3(B), dim3(kThreads), 0, graft::as_stream(stream), cand_parent,
                     cand_token, cand_score, cand_off, max_cand, budget, stage, anchor, anchor_token, err_flag);
  return graft::check_launch("prune_anchor");
}

extern "C" int graft_tail_cut(int B, int L, const int32_t *root_token, const int32_t *block_token,
                              const float *block_conf, float tau, int32_t *keep_len, int32_t *retrieval_root,
                              graft_stream stream) {
  using graft::fail;
  if (B < 0 || L < 1 || L >= GRAFT_MAX_NODES) return fail(GRAFT_EINVAL, "tail_cut: B=%d L=%d (1..%d)", B, L,
                                                           GRAFT_MAX_NODES - 1);
  if (B == 0) return GRAFT_OK;
  if (!root_token || !block_token || !block_conf || !keep_len || !retrieval_root)
    return fail(GRAFT_EINVAL, "tail_cut: NULL array");
  graft::clear_error();
  hipLaunchKernelGGL(tail_cut_kernel, dim3((B + 255) / 256), dim3(256), 0, graft::as_stream(stream), B, L, root_token,
                     block_token, block_conf, tau, keep_len, retrieval_root);
  return graft::check_launch("tail_cut");
}

extern "C" int graft_treegraft_node_count(int D, int W, int m, int mid_mask) {
  if (D < 0 || W < 1 || W > 64 || m < 1) return -1;
  return treegraft_count(D, W, m, mid_mask, GRAFT_MAX_CAND);
}

extern "C" int graft_treegraft_build(int B, int D, int W, int m, const int32_t *mid_mask, const int32_t *root_token,
                                     const int32_t *tok, const float *prob, const float *q, const int32_t *cand_off,
                                     int32_t *cand_parent, int32_t *cand_token, float *cand_score, int32_t *err_flag,
                                     graft_stream stream) {
  using graft::fail;
  if (B < 0 || D < 0 || D > 30 || W < 1 || W > 64 || m < 1 || m > GRAFT_MAX_CAND)
    return fail(GRAFT_EINVAL, "treegraft_build: B=%d D=%d W=%d (1..64) m=%d", B, D, W, m);
  if (B == 0) return GRAFT_OK;
  if (!mid_mask || !root_token || !cand_off || !cand_parent || !cand_token || !cand_score || !q ||
      (D > 0 && (!tok || !prob)))
    return fail(GRAFT_EINVAL, "treegraft_build: NULL array");
  graft::clear_error();
  hipLaunchKernelGGL(treegraft_kernel, dim3(B), dim3(kThreads), 0, graft::as_stream(stream), D, W, m, mid_mask,
                     root_token, tok, prob, q, cand_off, cand_parent, cand_token, cand_score, err_flag);
  return graft::check_launch("treegraft_build");
}
