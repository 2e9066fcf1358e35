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

// Largest b in [0, nb) with off[b] <= r (off non-decreasing, r < off[nb]).
__device__ int owner(const int32_t *off, int nb, int r) {
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Is update row r a verified node with in-range token and ids?
__device__ bool update_row_valid(int r, int V, int k, int B_upd, const int32_t *upd_n,
                                 const int32_t *upd_row_off, const int32_t *upd_token,
                                 const int32_t *upd_topk, int32_t *err, bool report) {
  int b = owner(upd_row_off, B_upd, r);
  int i = r - upd_row_off[b];
  if (i >= upd_n[b] || r >= upd_row_off[b + 1]) return false;  // padding row
  int t = upd_token[r];
  bool ok = t >= 0 && t < V;
  for (int j = 0; j < k; ++j) {
    int v = upd_topk[static_cast<size_t>(r) * k + j];
    ok = ok && v >= 0 && v < V;
  }
  if (!ok && report) graft::raise_flag(err, GRAFT_ERR_TOKEN);
  return ok;
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
  __shared__ int s_tp[GRAFT_MAX_TEMPLATE_ROWS];   // template parents, staged once
  __shared__ int s_own[GRAFT_MAX_TEMPLATE_ROWS];  // owning request of each template row
  __shared__ signed char s_depth[GRAFT_MAX_TEMPLATE_ROWS];
  __shared__ int s_maxdepth;
  const int tid = threadIdx.x;

  for (int h = tid; h < kSlots; h += kThreads) {
    s_key[h] = -1;
    s_val[h] = -1;
  }
  if (tid == 0) s_maxdepth = 0;
  for (int t = tid; t < tmpl_rows; t += kThreads) {
    s_tp[t] = tparent[t];
    s_own[t] = owner(toff, B, t);
  }
  for (int b = tid; b < B_upd; b += kThreads) {
    int cap = upd_row_off[b + 1] - upd_row_off[b];
    if (upd_n[b] < 0 || upd_n[b] > cap) graft::raise_flag(err, GRAFT_ERR_CAPACITY);
  }
  __syncthreads();

  // last writer wins: keep the largest row index per token
  for (int r = tid; r < upd_rows; r += kThreads) {
    if (update_row_valid(r, V, k, B_upd, upd_n, upd_row_off, upd_token, upd_topk, err, true))
      hash_insert(s_key, s_val, upd_token[r], r);
  }

  // template depths (request-local parents must precede their child)
  for (int t = tid; t < tmpl_rows; t += kThreads) {
    int b = s_own[t];
    int base = toff[b];
    int cur = t - base;
    int d = 1;
    bool ok = true;
    while (true) {
      int p = s_tp[base + cur];
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

  // copy the winning rows into the table (these rows are never read below)
  for (int r = tid; r < upd_rows; r += kThreads) {
    if (!update_row_valid(r, V, k, B_upd, upd_n, upd_row_off, upd_token, upd_topk, err, false))
      continue;
    int t = upd_token[r];
    if (hash_find(s_key, s_val, t) != r) continue;
    for (int j = 0; j < k; ++j)
      table[static_cast<size_t>(t) * k + j] = upd_topk[static_cast<size_t>(r) * k + j];
  }

  // expand the templates level by level
  const int maxd = s_maxdepth;
  for (int level = 1; level <= maxd; ++level) {
    for (int t = tid; t < tmpl_rows; t += kThreads) {
      if (s_depth[t] != level) continue;
      int b = s_own[t];
      int base = toff[b];
      int p = s_tp[t];
      int src = p < 0 ? root_token[b] : s_tok[base + p];
      int rank = trank[t];
      int tok = -1;
      if (rank < 0 || rank >= k) {
        graft::raise_flag(err, GRAFT_ERR_RANK);
      } else if (src >= 0 && src < V) {
        int w = hash_find(s_key, s_val, src);
        tok = w >= 0 ? upd_topk[static_cast<size_t>(w) * k + rank]
                     : table[static_cast<size_t>(src) * k + rank];
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
  if (B_upd < 0 || upd_rows < 0 || upd_rows > GRAFT_MAX_UPDATE_ROWS)
    return fail(GRAFT_EINVAL, "table_update_retrieve: B_upd=%d upd_rows=%d (max %d)", B_upd, upd_rows,
                GRAFT_MAX_UPDATE_ROWS);
  if (B < 0 || tmpl_rows < 0 || tmpl_rows > GRAFT_MAX_TEMPLATE_ROWS)
    return fail(GRAFT_EINVAL, "table_update_retrieve: B=%d tmpl_rows=%d (max %d)", B, tmpl_rows,
                GRAFT_MAX_TEMPLATE_ROWS);
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
