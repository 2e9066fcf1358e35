// Successor-table update and template retrieval.
//
// Graft page (arXiv:2605.20104 write-up), section 2, second step: the
// successor table lives in GPU memory, row t holds the k successors of t
// ranked highest by the target model, and a lookup is a single row index.
// Section 2, third step, and section 6: after verification every verified
// position -- accepted or rejected -- rewrites its token's row.
//
// One workgroup does both parts.  The update list is small (at most a few
// thousand rows: the nodes of one round's trees), so the kernel is bound by
// latency, not bandwidth: every global input is read in one round of loads,
// and template rows resolve in rounds, one per level, each a single
// dependent table read.  Same-token conflicts are resolved with an LDS hash
// map token -> largest row index; the winning rows are copied into the
// table.  Retrieval reads a row from the update list when its token was
// just updated and from the table otherwise, so it never reads memory this
// launch writes.
#include "common.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kSlots = 2 * GRAFT_MAX_UPDATE_ROWS;  // power of two, load <= 1/2
static_assert((kSlots & (kSlots - 1)) == 0, "hash size must be a power of two");

__device__ inline unsigned slot_of(int t) { return (static_cast<unsigned>(t) * 2654435761u) & (kSlots - 1); }

__device__ void hash_insert(int *keys, int *vals, int t, int row) {
  unsigned h = slot_of(t);
  for (int probe = 0; probe < kSlots; ++probe) {
    int old = atomicCAS(&keys[h], -1, t);
    if (old == -1 || old == t) {
      atomicMax(&vals[h], row);
      return;
    }
    h = (h + 1) & (kSlots - 1);
  }
}

__device__ int hash_find(const int *keys, const int *vals, int t) {
  unsigned h = slot_of(t);
  for (int probe = 0; probe < kSlots; ++probe) {
    int kk = keys[h];
    if (kk == t) return vals[h];
    if (kk == -1) return -1;
    h = (h + 1) & (kSlots - 1);
  }
  return -1;
}

// Largest b in [0, nb) with off[b] <= r (off non-decreasing, r < off[nb]);
// off is an LDS copy.
__device__ int owner(const int *off, int nb, int r) {
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Token at rank `rank` of src's successor row: from the update list when src
// was just updated (its winning row w), else from the table.  The table read
// is issued before the hash probe so the two latencies overlap; a stale row
// of an updated token is read and dropped.  Flags and returns -1 on a bad
// rank, source or entry (a parent without a token, src == -1, below the
// root, is not flagged again).
__device__ inline int lookup(const int32_t *table, const int32_t *upd_topk, const int *s_key, const int *s_val,
                             int V, int k, int src, int rank, bool below_root, int32_t *err) {
  if (rank < 0 || rank >= k) {
    graft::raise_flag(err, GRAFT_ERR_RANK);
    return -1;
  }
  if (src < 0 || src >= V) {
    if (!below_root || src != -1) graft::raise_flag(err, GRAFT_ERR_TOKEN);  // bad root or parent token
    return -1;
  }
  const int tv = table[static_cast<size_t>(src) * k + rank];
  const int w = hash_find(s_key, s_val, src);
  const int tok = w >= 0 ? upd_topk[static_cast<size_t>(w) * k + rank] : tv;
  if (tok < 0 || tok >= V) {
    graft::raise_flag(err, GRAFT_ERR_TOKEN);
    return -1;
  }
  return tok;
}

constexpr int kUpdPer = GRAFT_MAX_UPDATE_ROWS / kThreads;     // update rows per thread
constexpr int kTmplPer = GRAFT_MAX_TEMPLATE_ROWS / kThreads;  // template rows per thread
constexpr int kElemRegs = 8;  // update-list entries per thread held in registers (8192 in all)
constexpr int kMaxDepth = 127;  // deepest template level expanded

__global__ __launch_bounds__(kThreads) void update_retrieve_kernel(
    int32_t *__restrict__ table, int V, int k, int B_upd, const int32_t *__restrict__ upd_n,
    const int32_t *__restrict__ upd_row_off, int upd_rows, const int32_t *__restrict__ upd_token,
    const int32_t *__restrict__ upd_topk, int B, const int32_t *__restrict__ root_token,
    const int32_t *__restrict__ tparent, const int32_t *__restrict__ trank,
    const int32_t *__restrict__ toff, int tmpl_rows, int32_t *__restrict__ ret_token,
    int32_t *__restrict__ err) {
  __shared__ int s_key[kSlots];
  __shared__ int s_val[kSlots];
  __shared__ int s_utok[GRAFT_MAX_UPDATE_ROWS];             // token of a live, valid update row, else -1
  __shared__ unsigned char s_rowbad[GRAFT_MAX_UPDATE_ROWS];  // an id of the row is outside [0, V)
  __shared__ int s_tok[GRAFT_MAX_TEMPLATE_ROWS];
  __shared__ short s_round[GRAFT_MAX_TEMPLATE_ROWS];         // round a row was resolved in; -1 pending
  __shared__ signed char s_bad[GRAFT_MAX_TEMPLATE_ROWS];     // broken parent chain
  __shared__ int s_toff[GRAFT_MAX_BATCH + 1];
  __shared__ int s_root[GRAFT_MAX_BATCH];
  __shared__ int s_uoff[GRAFT_MAX_BATCH + 1];
  __shared__ int s_un[GRAFT_MAX_BATCH];
  __shared__ int s_straddle;  // a request's template rows span two wavefronts
  const int tid = threadIdx.x;
  const int n_elem = upd_rows * k;
  // Every argument in registers before the first load: fetched lazily, each
  // would cost a round trip of its own between the loads below.
  asm volatile("" ::"s"(table), "s"(upd_n), "s"(upd_row_off), "s"(upd_token), "s"(upd_topk), "s"(root_token),
               "s"(tparent), "s"(trank), "s"(toff), "s"(ret_token), "s"(err), "s"(V), "s"(k), "s"(B_upd),
               "s"(upd_rows), "s"(B), "s"(tmpl_rows));

  // ---- one round of coalesced loads into registers: offsets, roots, the
  // update list entry by entry, update tokens, template structure; only
  // then the LDS stores (a store between two loads makes the second wait
  // for the first).  B, B_upd <= kThreads: index kThreads of an offset array
  // (B + 1 entries) goes to thread 0.
  // The arrays of an empty part may be NULL (nothing reads them then):
  // their per-request entries count as zero.
  static_assert(GRAFT_MAX_BATCH <= kThreads, "one request per thread, plus the last offset");
  const bool have_t = toff && root_token, have_u = upd_row_off && upd_n;
  const int toff_a = have_t && tid <= B ? toff[tid] : 0;
  const int root_a = have_t && tid < B ? root_token[tid] : 0;
  const int uoff_a = have_u && tid <= B_upd ? upd_row_off[tid] : 0;
  const int un_a = have_u && tid < B_upd ? upd_n[tid] : 0;
  const int toff_b = have_t && tid == 0 && B == kThreads ? toff[kThreads] : 0;
  const int uoff_b = have_u && tid == 0 && B_upd == kThreads ? upd_row_off[kThreads] : 0;
  int ev[kElemRegs];
#pragma unroll
  for (int q = 0; q < kElemRegs; ++q) {
    const int e = q * kThreads + tid;
    ev[q] = e < n_elem ? upd_topk[e] : 0;
  }
  int utok[kUpdPer];
#pragma unroll
  for (int u = 0; u < kUpdPer; ++u) {
    const int r = u * kThreads + tid;
    utok[u] = r < upd_rows ? upd_token[r] : -1;
  }
  int tpar[kTmplPer], trk[kTmplPer];
#pragma unroll
  for (int i = 0; i < kTmplPer; ++i) {
    const int t = i * kThreads + tid;
    tpar[i] = t < tmpl_rows ? tparent[t] : -1;
    trk[i] = t < tmpl_rows ? trank[t] : -1;
  }
  __builtin_amdgcn_sched_barrier(0);  // the loads above stay ahead of the stores below
  for (int h = tid; h < kSlots; h += kThreads) {
    s_key[h] = -1;
    s_val[h] = -1;
  }
  if (tid <= B) s_toff[tid] = toff_a;
  if (tid < B) s_root[tid] = root_a;
  if (tid <= B_upd) s_uoff[tid] = uoff_a;
  if (tid < B_upd) s_un[tid] = un_a;
  if (tid == 0 && B == kThreads) s_toff[kThreads] = toff_b;
  if (tid == 0 && B_upd == kThreads) s_uoff[kThreads] = uoff_b;
  if (tid == 0) s_straddle = tmpl_rows > kThreads ? 1 : 0;
#pragma unroll
  for (int u = 0; u < kUpdPer; ++u) {
    const int r = u * kThreads + tid;
    if (r < upd_rows) s_rowbad[r] = 0;
  }
  __syncthreads();

  // ---- ids outside the vocabulary mark their row; request capacities;
  // template rows: owner, and the link to a request-local parent, which must
  // precede its child
#pragma unroll
  for (int q = 0; q < kElemRegs; ++q) {
    const int e = q * kThreads + tid;
    if (e < n_elem && (ev[q] < 0 || ev[q] >= V)) s_rowbad[e / k] = 1;
  }
  for (int e = kElemRegs * kThreads + tid; e < n_elem; e += kThreads) {
    const int v = upd_topk[e];
    if (v < 0 || v >= V) s_rowbad[e / k] = 1;
  }
  for (int b = tid; b < B_upd; b += kThreads) {
    const int cap = s_uoff[b + 1] - s_uoff[b];
    const int nb = s_un[b];
    if (nb < 0 || nb > cap) graft::raise_flag(err, GRAFT_ERR_CAPACITY);
  }
  int town[kTmplPer], tbase[kTmplPer];
  unsigned pend = 0;
#pragma unroll
  for (int i = 0; i < kTmplPer; ++i) {
    const int t = i * kThreads + tid;
    town[i] = 0;
    tbase[i] = 0;
    if (t < tmpl_rows) {
      town[i] = owner(s_toff, B, t);
      tbase[i] = s_toff[town[i]];
      // rows before tmpl_off[0] belong to no request: skipped, not flagged
      const bool in_req = t >= tbase[i];
      const bool link_ok = in_req & (tpar[i] < t - tbase[i]);
      if (in_req & !link_ok) graft::raise_flag(err, GRAFT_ERR_PARENT);
      s_round[t] = link_ok ? -1 : 0;
      s_bad[t] = link_ok ? 0 : 1;
      if (link_ok) pend |= 1u << i;
      if (in_req & ((tbase[i] >> 6) != (t >> 6))) s_straddle = 1;
    }
  }
  __syncthreads();

  // ---- update rows of verified nodes with valid ids; last writer wins: keep
  // the largest row index per token
#pragma unroll
  for (int u = 0; u < kUpdPer; ++u) {
    const int r = u * kThreads + tid;
    if (r < upd_rows) {
      const int b = owner(s_uoff, B_upd, r);
      // a node of request b (not a padding row, not a row before upd_row_off[0])
      const bool live = (r >= s_uoff[b]) & (r - s_uoff[b] < s_un[b]) & (r < s_uoff[b + 1]);
      int t = -1;
      if (live) {
        if (utok[u] >= 0 && utok[u] < V && !s_rowbad[r]) t = utok[u];
        else graft::raise_flag(err, GRAFT_ERR_TOKEN);
      }
      s_utok[r] = t;
      if (t >= 0) hash_insert(s_key, s_val, t, r);
    }
  }
  __syncthreads();

  // ---- expand the templates: a row is resolved in the round after its
  // parent, so round d resolves depth d.  When every request's rows sit in
  // one wavefront (at most 1024 rows), each wavefront runs its own rounds
  // and takes parent tokens by lane shuffle; otherwise parents are read
  // from LDS between workgroup barriers.
  if (!s_straddle) {
    const int lane = tid & 63;
    const int p = tpar[0];
    const int pl = p >= 0 ? ((tbase[0] + p) & 63) : lane;  // parent's lane
    bool pending = pend & 1u;
    bool bad = tid < tmpl_rows && !pending;  // broken parent link
    int tok = -1;
    for (int round = 1; round <= kMaxDepth; ++round) {
      if (__builtin_amdgcn_ballot_w64(pending) == 0) break;
      const int ptok = __shfl(tok, pl);
      const int pst = __shfl((pending ? 1 : 0) | (bad ? 2 : 0), pl);
      if (pending && (p < 0 || !(pst & 1))) {
        if (p >= 0 && (pst & 2)) {
          graft::raise_flag(err, GRAFT_ERR_PARENT);
          bad = true;
        } else {
          tok = lookup(table, upd_topk, s_key, s_val, V, k, p < 0 ? s_root[town[0]] : ptok, trk[0], p >= 0, err);
        }
        pending = false;
      }
    }
    if (pending) graft::raise_flag(err, GRAFT_ERR_PARENT);  // deeper than kMaxDepth levels
    if (tid < tmpl_rows) ret_token[tid] = (!pending && !bad) ? tok : -1;
  } else {
    for (int round = 1; round <= kMaxDepth; ++round) {
#pragma unroll
      for (int i = 0; i < kTmplPer; ++i) {
        if (!(pend & (1u << i))) continue;
        const int t = i * kThreads + tid;
        const int p = tpar[i];
        const int pr = p < 0 ? 0 : s_round[tbase[i] + p];
        if (p >= 0 && (pr < 0 || pr >= round)) continue;  // parent not resolved before this round
        const bool bad = p >= 0 && s_bad[tbase[i] + p];
        int tok = -1;
        if (bad) {
          graft::raise_flag(err, GRAFT_ERR_PARENT);
        } else {
          const int src = p < 0 ? s_root[town[i]] : s_tok[tbase[i] + p];
          tok = lookup(table, upd_topk, s_key, s_val, V, k, src, trk[i], p >= 0, err);
        }
        s_tok[t] = tok;
        s_bad[t] = bad ? 1 : 0;
        s_round[t] = static_cast<short>(round);
        pend &= ~(1u << i);
      }
      if (!__syncthreads_or(pend != 0)) break;
    }
    if (pend) graft::raise_flag(err, GRAFT_ERR_PARENT);  // deeper than kMaxDepth levels
#pragma unroll
    for (int i = 0; i < kTmplPer; ++i) {
      const int t = i * kThreads + tid;
      if (t < tmpl_rows)
        ret_token[t] = (!(pend & (1u << i)) && !s_bad[t] && s_round[t] > 0) ? s_tok[t] : -1;
    }
  }

  // ---- copy the winning rows into the table, entry by entry (retrieval above
  // read these tokens' rows from the update list)
#pragma unroll
  for (int q = 0; q < kElemRegs; ++q) {
    const int e = q * kThreads + tid;
    if (e < n_elem) {
      const int r = e / k;
      const int t = s_utok[r];
      if (t >= 0 && hash_find(s_key, s_val, t) == r) table[static_cast<size_t>(t) * k + (e - r * k)] = ev[q];
    }
  }
  for (int e = kElemRegs * kThreads + tid; e < n_elem; e += kThreads) {
    const int r = e / k;
    const int t = s_utok[r];
    if (t >= 0 && hash_find(s_key, s_val, t) == r) table[static_cast<size_t>(t) * k + (e - r * k)] = upd_topk[e];
  }
}

}  // namespace

extern "C" int graft_table_update_retrieve(int32_t *table, int V, int k, int B_upd,
                                           const int32_t *upd_n, const int32_t *upd_row_off,
                                           int upd_rows, const int32_t *upd_token,
                                           const int32_t *upd_topk, int B,
                                           const int32_t *root_token, const int32_t *tmpl_parent,
                                           const int32_t *tmpl_rank, const int32_t *tmpl_off,
                                           int tmpl_rows, int32_t *ret_token, int32_t *err_flag,
                                           graft_stream stream) {
  using graft::fail;
  if (V <= 0 || k < 1 || k > GRAFT_MAX_K) return fail(GRAFT_EINVAL, "table_update_retrieve: V=%d k=%d", V, k);
  if (!table) return fail(GRAFT_EINVAL, "table_update_retrieve: table is NULL");
  if (B_upd < 0 || B_upd > GRAFT_MAX_BATCH || upd_rows < 0 || upd_rows > GRAFT_MAX_UPDATE_ROWS)
    return fail(GRAFT_EINVAL, "table_update_retrieve: B_upd=%d (max %d) upd_rows=%d (max %d)", B_upd,
                GRAFT_MAX_BATCH, upd_rows, GRAFT_MAX_UPDATE_ROWS);
  if (B < 0 || B > GRAFT_MAX_BATCH || tmpl_rows < 0 || tmpl_rows > GRAFT_MAX_TEMPLATE_ROWS)
    return fail(GRAFT_EINVAL, "table_update_retrieve: B=%d (max %d) tmpl_rows=%d (max %d)", B, GRAFT_MAX_BATCH,
                tmpl_rows, GRAFT_MAX_TEMPLATE_ROWS);
  if (B_upd == 0) upd_rows = 0;
  if (B == 0) tmpl_rows = 0;
  if (upd_rows > 0 && (!upd_n || !upd_row_off || !upd_token || !upd_topk))
    return fail(GRAFT_EINVAL, "table_update_retrieve: NULL update array");
  if (tmpl_rows > 0 && (!root_token || !tmpl_parent || !tmpl_rank || !tmpl_off || !ret_token))
    return fail(GRAFT_EINVAL, "table_update_retrieve: NULL template array");
  if (upd_rows == 0 && tmpl_rows == 0) return GRAFT_OK;
  graft::clear_error();
  hipLaunchKernelGGL(update_retrieve_kernel, dim3(1), dim3(kThreads), 0, graft::as_stream(stream), table, V,
                     k, B_upd, upd_n, upd_row_off, upd_rows, upd_token, upd_topk, B, root_token,
                     tmpl_parent, tmpl_rank, tmpl_off, tmpl_rows, ret_token, err_flag);
  return graft::check_launch("table_update_retrieve");
}
