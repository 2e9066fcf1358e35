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
// latency, not bandwidth.  Same-token conflicts are resolved with an LDS
// hash map token -> largest row index; the winning rows are copied into
// the table.  Retrieval then reads a row from the update list when its
// token was just updated and from the table otherwise, so it never reads
// memory this launch writes.
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


__global__ __launch_bounds__(kThreads) void update_retrieve_kernel(
    int32_t *__restrict__ table, int V, int k, int B_upd, const int32_t *__restrict__ upd_n,
    const int32_t *__restrict__ upd_row_off, int upd_rows, const int32_t *__restrict__ upd_token,
    const int32_t *__restrict__ upd_topk, int B, const int32_t *__restrict__ root_token,
    const int32_t *__restrict__ tparent, const int32_t *__restrict__ trank,
    const int32_t *__restrict__ toff, int tmpl_rows, int32_t *__restrict__ ret_token,
    int32_t *__restrict__ err) {
  __shared__ int s_key[kSlots];
  __shared__ int s_val[kSlots];
  __shared__ int s_tok[GRAFT_MAX_TEMPLATE_ROWS];
  __shared__ int s_tp[GRAFT_MAX_TEMPLATE_ROWS];    // template parents
  __shared__ int s_own[GRAFT_MAX_TEMPLATE_ROWS];   // owning request of each template row
  __shared__ int s_utok[GRAFT_MAX_UPDATE_ROWS];    // token of a valid update row, else -1
  __shared__ signed char s_rank[GRAFT_MAX_TEMPLATE_ROWS];
  __shared__ signed char s_depth[GRAFT_MAX_TEMPLATE_ROWS];
  __shared__ int s_toff[GRAFT_MAX_BATCH + 1];
  __shared__ int s_root[GRAFT_MAX_BATCH];
  __shared__ int s_uoff[GRAFT_MAX_BATCH + 1];
  __shared__ int s_un[GRAFT_MAX_BATCH];
  __shared__ int s_maxdepth;
  const int tid = threadIdx.x;

  // ---- one round of loads: offsets, roots, template structure
  for (int h = tid; h < kSlots; h += kThreads) {
    s_key[h] = -1;
    s_val[h] = -1;
  }
  if (tid == 0) s_maxdepth = 0;
  for (int b = tid; b <= B; b += kThreads) {
    s_toff[b] = toff[b];
    if (b < B) s_root[b] = root_token[b];
  }
  for (int b = tid; b <= B_upd; b += kThreads) {
    s_uoff[b] = upd_row_off[b];
    if (b < B_upd) s_un[b] = upd_n[b];
  }
  for (int t = tid; t < tmpl_rows; t += kThreads) {
    s_tp[t] = tparent[t];
    s_rank[t] = static_cast<signed char>(min(max(trank[t], -1), 127));
  }
  __syncthreads();
  for (int t = tid; t < tmpl_rows; t += kThreads) s_own[t] = owner(s_toff, B, t);
  for (int b = tid; b < B_upd; b += kThreads) {
    const int cap = s_uoff[b + 1] - s_uoff[b];
    const int nb = s_un[b];
    if (nb < 0 || nb > cap) graft::raise_flag(err, GRAFT_ERR_CAPACITY);
  }

  // ---- update rows: validity (verified node, token and ids in range);
  // last writer wins: keep the largest row index per token
  for (int r = tid; r < upd_rows; r += kThreads) {
    const int b = owner(s_uoff, B_upd, r);
    const int i = r - s_uoff[b];
    const int nb = s_un[b];
    int tok = -1;
    if (i < nb && r < s_uoff[b + 1]) {  // not a padding row
      const int t = upd_token[r];
      bool ok = t >= 0 && t < V;
      for (int j = 0; j < k; ++j) {
        const int v = upd_topk[static_cast<size_t>(r) * k + j];
        ok = ok && v >= 0 && v < V;
      }
      if (!ok) graft::raise_flag(err, GRAFT_ERR_TOKEN);
      else tok = t;
    }
    s_utok[r] = tok;
    if (tok >= 0) hash_insert(s_key, s_val, tok, r);
  }
  __syncthreads();

  // ---- template depths (request-local parents must precede their child)
  for (int t = tid; t < tmpl_rows; t += kThreads) {
    const int base = s_toff[s_own[t]];
    int cur = t - base;
    int d = 1;
    bool ok = true;
    while (true) {
      const int p = s_tp[base + cur];
      if (p < 0) break;
      if (p >= cur) {
        ok = false;
        break;
      }
      cur = p;
      ++d;
    }
    if (!ok || d > 127) {
      graft::raise_flag(err, GRAFT_ERR_PARENT);
      s_depth[t] = -1;
    } else {
      s_depth[t] = static_cast<signed char>(d);
      atomicMax(&s_maxdepth, d);
    }
  }
  __syncthreads();

  // ---- expand the templates level by level; a just-updated token's row is
  // read from the update list, any other from the table (never memory this
  // launch writes)
  const int maxd = s_maxdepth;
  for (int level = 1; level <= maxd; ++level) {
    for (int t = tid; t < tmpl_rows; t += kThreads) {
      if (s_depth[t] != level) continue;
      const int b = s_own[t];
      const int base = s_toff[b];
      const int p = s_tp[t];
      const int src = p < 0 ? s_root[b] : s_tok[base + p];
      const int rank = s_rank[t];
      int tok = -1;
      if (rank < 0 || rank >= k) {
        graft::raise_flag(err, GRAFT_ERR_RANK);
      } else if (src >= 0 && src < V) {
        const int w = hash_find(s_key, s_val, src);
        tok = w >= 0 ? upd_topk[static_cast<size_t>(w) * k + rank] : table[static_cast<size_t>(src) * k + rank];
        if (tok < 0 || tok >= V) {
          graft::raise_flag(err, GRAFT_ERR_TOKEN);
          tok = -1;
        }
      } else if (p < 0 || src != -1) {
        graft::raise_flag(err, GRAFT_ERR_TOKEN);  // bad root (or bad parent token)
      }
      s_tok[t] = tok;
    }
    __syncthreads();
  }
  for (int t = tid; t < tmpl_rows; t += kThreads) ret_token[t] = s_depth[t] > 0 ? s_tok[t] : -1;

  // ---- copy the winning rows into the table (rows read above come from the
  // update list for these tokens, so the order does not matter)
  for (int r = tid; r < upd_rows; r += kThreads) {
    const int t = s_utok[r];
    if (t < 0 || hash_find(s_key, s_val, t) != r) continue;
    for (int j = 0; j < k; ++j)
      table[static_cast<size_t>(t) * k + j] = upd_topk[static_cast<size_t>(r) * k + j];
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
