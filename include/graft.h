/*
 * graft.h -- C ABI of libgraft: one round of tree speculative decoding on
 * an AMD Instinct MI355X (gfx950).
 *
 * A round (Graft page = write-up of arXiv:2605.20104, section 2; TreeGraft
 * page = reading notes on arXiv:2608.26112, section 3):
 *   graft_table_update_retrieve  previous round's verified positions rewrite
 *                                their successor-table rows; the current
 *                                token's retrieval template is expanded
 *   graft_build_tree             draft selection + retrieved nodes, flatten,
 *                                depth / positions / ancestor mask
 *   graft_prune_anchor           (trees pruned at a checkpoint) the node the
 *                                retrieved nodes hang under, and its token,
 *                                the retrieval root
 *   graft_tree_attention         tree-masked GQA attention over the KV cache
 *   graft_lmhead_topk            logits = hidden . W^T and per-row top-k
 *                                (weights packed once by graft_lmhead_pack)
 *   graft_accept                 deepest greedily accepted path + bonus token
 *   graft_lmhead_topk_sample,    (temperature T > 0) one draw per row by
 *   graft_accept_sampled         Gumbel-max with the noise as an input, and
 *                                acceptance of the first matching child
 *   graft_treegraft_build        (TreeGraft) the shared tree of a small and a
 *                                mid drafter, upstream of graft_build_tree
 *   graft_kv_compact             (round chaining) the accepted path's K/V
 *                                moves to the front of the tree slots, the
 *                                context advances, the bonus becomes the
 *                                next root
 *
 * Conventions shared by every entry point
 *  - Pointers marked (device) are device memory owned by the caller; the
 *    library never allocates, frees or keeps them.  (host) pointers are
 *    read or written before the call returns.
 *  - Every device entry point is asynchronous on `stream` (a hipStream_t
 *    passed as void*; NULL = the null stream) and never synchronises with
 *    the host.
 *  - Return value: GRAFT_OK, or a negative status when a host-checkable
 *    argument is wrong (nothing is launched) or a launch failed;
 *    graft_last_error() then describes it (per thread).
 *  - Data-dependent faults found on the device (a token outside [0, V), a
 *    parent that does not precede its child, ...) never cause an
 *    out-of-bounds access: the kernel ORs a GRAFT_ERR_* bit into *err_flag
 *    (device int32, may be NULL) and produces in-bounds but unspecified
 *    values for the affected request.  The caller clears *err_flag.
 *  - Tree batches use a padded row layout: request b owns rows
 *    row_off[b] .. row_off[b+1]-1 (capacity <= 64) of every per-node array,
 *    and its node i (i < n[b]) is row row_off[b] + i.  row_off is
 *    non-decreasing.  Parent indices are request-local (root = node 0,
 *    parent -1).
 *  - Arrays of bf16 or fp32 values that a kernel moves 16 bytes at a time
 *    (hidden states, weights, logits, noise, Q, K/V caches, attention
 *    output, the tree-attention workspace) must be 16-byte aligned, and
 *    K/V offsets and strides multiples of 8 elements; every PyTorch
 *    allocation is aligned.  A
 *    misaligned pointer or stride returns GRAFT_EINVAL; a misaligned kv_off
 *    entry (device data) raises GRAFT_ERR_ALIGN and skips that request.
 *  - Integer results are exact; ties in any ranking go to the lower index.
 *    A NaN score or logit ranks below every number (NaNs tie with each
 *    other); -0 and +0 tie.
 *  - bf16 tensors are raw bfloat16 bit patterns (uint16).
 */
#ifndef GRAFT_H
#define GRAFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t graft_bf16;
typedef void *graft_stream;

#define GRAFT_MAX_NODES 64
#define GRAFT_MAX_K 16
/* Largest vocabulary the top-k paths take: their sort keys hold a token id
 * in 30 bits. */
#define GRAFT_MAX_V ((1 << 30) - 1)
#define GRAFT_MAX_CAND 2048
#define GRAFT_MAX_UPDATE_ROWS 4096
#define GRAFT_MAX_TEMPLATE_ROWS 4096
#define GRAFT_MAX_BATCH 1024 /* requests per table update / retrieval call */
#define GRAFT_ATTN_MAX_BATCH 8192 /* requests per tree attention call */

/* return status */
#define GRAFT_OK 0
#define GRAFT_EINVAL (-1)       /* bad argument / shape; nothing launched */
#define GRAFT_EUNSUPPORTED (-2) /* valid but not built (e.g. head dim 96) */
#define GRAFT_EHIP (-3)         /* a HIP launch failed */
#define GRAFT_EIO (-4)          /* a file could not be opened, read or written */

/* device error-flag bits */
#define GRAFT_ERR_TOKEN 1      /* token or successor id outside [0, V) */
#define GRAFT_ERR_PARENT 2     /* parent not earlier than its child / no root */
#define GRAFT_ERR_NOT_CLOSED 4 /* a kept draft node's parent was pruned */
#define GRAFT_ERR_CAPACITY 8   /* tree larger than its rows or 64 nodes, or a
                                  length above the bound given to the call */
#define GRAFT_ERR_RANK 16      /* template rank outside [0, k) */
#define GRAFT_ERR_ALIGN 32     /* a K/V base offset (kv_off) not a multiple of
                                  8 elements */

/* node source codes written by graft_build_tree */
#define GRAFT_SRC_ROOT 0
#define GRAFT_SRC_DRAFT 1
#define GRAFT_SRC_RETRIEVED 2
#define GRAFT_SRC_REPLACED 3

/* graft_build_tree modes */
#define GRAFT_TREE_PRUNE 0          /* top-budget draft nodes + retrieved nodes */
#define GRAFT_TREE_STATIC_REPLACE 1 /* top-budget draft nodes, low-score ones
                                       swapped for table successors */
#define GRAFT_TREE_TAIL 2           /* block draft: confident prefix kept, the
                                       freed slots from retrieval under it */

const char *graft_last_error(void);
int graft_version(void);

/*
 * Successor-table update, then template retrieval.
 * Graft page, section 2 (second step: a GPU-resident table whose row t
 * lists t's most likely successors; retrieval expands a stage-adaptive
 * template from the current token by row lookups) and section 2 third step
 * plus section 6 (every verified position, accepted or rejected, rewrites
 * its token's row with the target's most likely successors).
 *
 * table       (device) int32 [V, k], updated in place.
 * Update: the verified nodes of B_upd requests in the padded row layout
 *   (upd_n [B_upd], upd_row_off [B_upd+1], device); upd_token [rows] and
 *   upd_topk [rows, k] (device, row-major, the top-k ids of each row).  For
 *   node r the whole row table[upd_token[r]] becomes upd_topk[r]; when
 *   several nodes carry the same token the largest row index wins.
 *   upd_rows (host) = upd_row_off[B_upd] <= GRAFT_MAX_UPDATE_ROWS; rows
 *   before upd_row_off[0] belong to no request and are ignored.
 *   A node whose token or ids fall outside [0, V) is skipped (ERR_TOKEN).
 * Retrieval (after the update): request b's template nodes are
 *   tmpl_off[b] .. tmpl_off[b+1]-1 (device) with request-local template
 *   parents tmpl_parent (-1 = the root, otherwise an earlier node) and ranks
 *   tmpl_rank in [0, k); node t gets
 *     ret_token[t] = table'[token of its parent (root_token[b] for -1)][rank]
 *   where table' is the updated table.  tmpl_rows (host) = tmpl_off[B] <=
 *   GRAFT_MAX_TEMPLATE_ROWS.  Invalid links yield ret_token = -1 with
 *   ERR_PARENT / ERR_RANK / ERR_TOKEN.  Rows before tmpl_off[0] belong to
 *   no request: ret_token = -1, nothing flagged.
 * Either part may be empty (B_upd = 0 or upd_rows = 0; B = 0 or
 * tmpl_rows = 0).  B, B_upd <= GRAFT_MAX_BATCH (their offsets are staged in
 * LDS); larger batches return GRAFT_EINVAL.  One workgroup; calls that
 * overlap on a table race.
 */
int graft_table_update_retrieve(int32_t *table, int V, int k,
                                int B_upd, const int32_t *upd_n, const int32_t *upd_row_off,
                                int upd_rows, const int32_t *upd_token, const int32_t *upd_topk,
                                int B, const int32_t *root_token, const int32_t *tmpl_parent,
                                const int32_t *tmpl_rank, const int32_t *tmpl_off, int tmpl_rows,
                                int32_t *ret_token, int32_t *err_flag, graft_stream stream);

/*
 * Successor-table checkpoint.  The table is the only state a round leaves
 * besides the KV cache, and a warmed table is kept across rounds (Graft
 * page, section 6: warm-up fills the table, later rounds keep updating it).
 * File: 32-byte header ("GRAFTTB1", V and k as little-endian int64, the
 * 64-bit FNV-1a hash of the payload), then table [V, k] int32 row-major,
 * little-endian.
 * graft_table_save copies table (device) to the host on `stream`, waits for
 * the stream, and writes the file under path + ".tmp", renamed to path when
 * whole.  graft_table_load reads the file, checks the magic, V and k (which
 * must equal the arguments), the length, the hash and that every entry lies
 * in [0, V), and only then copies the rows to table (device) on `stream`
 * and waits for it; on any error table is left untouched.
 * 1 <= k <= GRAFT_MAX_K.  Errors: GRAFT_EINVAL (arguments, or a file that is
 * not this table), GRAFT_EIO (open, read, write, rename), GRAFT_EHIP (copy).
 */
int graft_table_save(const char *path, int V, int k, const int32_t *table, graft_stream stream);
int graft_table_load(const char *path, int V, int k, int32_t *table, graft_stream stream);

/*
 * Tree construction and flattening for B requests.
 * Draft selection by cumulative score and global prune (TreeGraft page,
 * section 3 and section 4 "How"); Graft's stage budgets and retrieval fill
 * (Graft page, section 2, second step); flatten + tree positions + mask
 * (Graft page, section 2, third step); static-tree replacement for batched
 * serving (Graft page, section 4, serving paragraph).
 *
 * Candidates of request b: cand_off[b] .. cand_off[b+1]-1 (device) of
 *   cand_parent (request-local, candidate 0 is the root with parent -1,
 *   others point to an earlier candidate), cand_token, cand_score (fp32
 *   cumulative score, non-increasing along paths).  max_cand (host) bounds
 *   every request's candidate count, <= GRAFT_MAX_CAND.
 * budget[b] (device): draft nodes kept, root included: the root plus the
 *   budget-1 best other candidates by (score desc, index asc).
 * mode GRAFT_TREE_PRUNE: the request's retrieved nodes ret_off[b] ..
 *   ret_off[b+1]-1 (ret_token, ret_parent = template parents, -1 = the
 *   anchor) are appended after the kept draft nodes.  ret_* may be NULL
 *   for none.  ret_anchor (device int32 [B], may be NULL = every request's
 *   root): the candidate the retrieved nodes hang under, e.g. from
 *   graft_prune_anchor; one that is not kept flags ERR_NOT_CLOSED and the
 *   root is used.
 * mode GRAFT_TREE_STATIC_REPLACE: no retrieved nodes; a kept draft node
 *   with score < replace_thresh that is the j-th (0-based, by index) such
 *   child of its parent takes token table[token(parent)][j] when j < k
 *   (parent token after its own replacement), source GRAFT_SRC_REPLACED.
 *   table (device int32 [V, k]) is read only in this mode.
 * mode GRAFT_TREE_TAIL (Graft page, section 7, Graft-TAIL on block drafts;
 *   the thresholds and shapes are this library's reading): the candidates
 *   are the root and a block draft, cand_score = the drafter's confidence
 *   per token; candidates 0..K are kept, where K + 1 is the first index
 *   >= 1 with cand_score < replace_thresh (NaN counts as below), and the
 *   first budget[b] - (K + 1) retrieved rows of the request follow, their
 *   template parent -1 meaning node K (the deepest kept node).  The rows
 *   must be a template whose first rows are the smaller templates (as
 *   graft_make_template's are), expanded from graft_tail_cut's
 *   retrieval_root.  budget[b] = 1 + block length keeps the slot count.
 * Output per request (device, padded row layout given by row_off [B+1]):
 *   n_out[b]; parent, token, depth, pos = ctx_len[b] + depth (int32),
 *   mask (uint64: bit j set iff node j is the node or its ancestor) and
 *   src (int8).  Flattened order: kept draft nodes in ascending candidate
 *   index, then retrieved nodes in template order.  Rows past n_out[b]
 *   get parent = token = depth = pos = -1, mask = 0, src = -1.
 * A tree over min(64, capacity) nodes, or over max_cand candidates, gives
 * n_out[b] = 0 and ERR_CAPACITY.
 */
int graft_build_tree(int B, int mode,
                     const int32_t *cand_parent, const int32_t *cand_token, const float *cand_score,
                     const int32_t *cand_off, int max_cand, const int32_t *budget,
                     const int32_t *ret_token, const int32_t *ret_parent, const int32_t *ret_off,
                     const int32_t *ret_anchor, const int32_t *table, int V, int k, float replace_thresh,
                     const int32_t *ctx_len, const int32_t *row_off,
                     int32_t *n_out, int32_t *parent, int32_t *token, int32_t *depth,
                     int32_t *pos, uint64_t *mask, int8_t *src, int32_t *err_flag,
                     graft_stream stream);

/*
 * Retrieval anchor of trees pruned at a checkpoint (Graft page, section 2,
 * second step: the drafter's tree is checked at depths 0, 1 and 5 by the
 * current best path's cumulative confidence; when pruning triggers, the
 * retrieval tree is expanded from the token generated up to that point).
 * This library's reading: the best path at checkpoint depth c ends at the
 * candidate of depth c with the highest cumulative score (ties: lower
 * index; c is capped at the deepest candidate depth); the anchor is that
 * candidate when graft_build_tree's budget keeps it, else its deepest kept
 * ancestor.  c <= 0 anchors at the root.
 * Candidates, max_cand and budget (device) as in graft_build_tree;
 * stage (device int32 [B]) = each request's checkpoint depth c.
 * Outputs (device int32 [B]): anchor[b] = the request-local candidate index
 * (pass as graft_build_tree's ret_anchor) and anchor_token[b] = its token
 * (pass as graft_table_update_retrieve's root_token).  A malformed candidate
 * list flags ERR_CAPACITY / ERR_PARENT and anchors at the root.
 */
int graft_prune_anchor(int B, const int32_t *cand_parent, const int32_t *cand_token, const float *cand_score,
                       const int32_t *cand_off, int max_cand, const int32_t *budget, const int32_t *stage,
                       int32_t *anchor, int32_t *anchor_token, int32_t *err_flag, graft_stream stream);

/*
 * TreeGraft's shared draft tree from a small and a mid drafter (TreeGraft
 * page, section 3: at step k the frontier is the best W nodes of the pool by
 * cumulative score s, the product of edge scores from the root, and each
 * frontier node gets m children; section 4 "Where": a mid-drafter step's
 * pool is every node it has not yet visited, ranked by its own path score,
 * and visits the pool; a small-drafter step's pool is the previous step's
 * new nodes with their stored scores; "How": children are appended without
 * overwriting; the global prune to Bver is graft_build_tree afterwards).
 * The drafters and the schedule ("When") are out of scope and come in:
 *   mid_mask[b] (device int32): bit k set = step k is a mid-drafter step;
 *   tok, prob (device [B][D][W][m], int32 / fp32): the step's drafter output
 *     for the j-th best frontier node, child c (children are created in that
 *     order, numbered after every earlier node);
 *   q (device fp32, the candidate layout): q[cand_off[b] + v] is the mid
 *     drafter's probability of the edge into node v; its path score is
 *     r(v) = fl(r(parent) * q[v]), r(root) = 1.
 * A child of frontier node f gets score fl(s(f) * prob); ties in ranking go
 * to the lower node index.  Output per request at cand_off[b] (device
 * [B+1]): cand_parent (root -1), cand_token (root = root_token[b]),
 * cand_score = s, in creation order (topological): the candidate arrays of
 * graft_build_tree.  cand_off[b+1] - cand_off[b] must equal
 * graft_treegraft_node_count(D, W, m, mid_mask[b]) (a host helper: the
 * count depends on the sizes and schedule only; -1 for invalid sizes or
 * more than GRAFT_MAX_CAND nodes), else the request is flagged ERR_CAPACITY
 * and left unwritten.  1 <= W <= 64, D <= 30.
 */
int graft_treegraft_node_count(int D, int W, int m, int mid_mask);
int graft_treegraft_build(int B, int D, int W, int m, const int32_t *mid_mask, const int32_t *root_token,
                          const int32_t *tok, const float *prob, const float *q, const int32_t *cand_off,
                          int32_t *cand_parent, int32_t *cand_token, float *cand_score, int32_t *err_flag,
                          graft_stream stream);

/*
 * Graft-TAIL cut (Graft page, section 7): per request b, keep_len[b] = the
 * number of leading block tokens with confidence >= tau (NaN counts as
 * below) and retrieval_root[b] = the token of the deepest kept node, i.e.
 * block_token[b * L + keep_len[b] - 1], or root_token[b] when none is kept:
 * the root to pass to graft_table_update_retrieve before graft_build_tree
 * in mode GRAFT_TREE_TAIL.  block_token [B, L], block_conf [B, L] (fp32),
 * root_token [B], outputs [B]: device.  1 <= L <= 63.
 */
int graft_tail_cut(int B, int L, const int32_t *root_token, const int32_t *block_token,
                   const float *block_conf, float tau, int32_t *keep_len, int32_t *retrieval_root,
                   graft_stream stream);

/*
 * Tree-masked grouped-query attention (Graft page, section 2, third step:
 * one parallel verification of the flattened tree with its tree mask;
 * TreeGraft page, section 3 and section 7 item 1: tree attention).
 *
 * For request b, node i < n[b], query head h (kv head h / (Hq/Hkv)):
 *   out = softmax(scale * q . K^T) V  over cache slots 0 .. ctx_len[b]-1
 *   and the tree slots ctx_len[b] + j with bit j of mask[row_off[b]+i].
 * q, out  (device) bf16 [rows, Hq, d] with row = row_off[b] + i.
 * kcache, vcache (device) bf16: slot s of kv head h of request b at
 *   element kv_off[b] + h * kv_head_stride + s * d; tree node j's key and
 *   value sit at slot ctx_len[b] + j.
 * ctx_len, n (device int32 [B]); max_ctx, max_n (host) bound them (work
 *   and workspace sizing); a request above a bound is skipped with
 *   ERR_CAPACITY.  B <= GRAFT_ATTN_MAX_BATCH, and the key chunks
 *   B * Hkv * ceil(max_n * (Hq / Hkv) / rows per workgroup) *
 *   ceil((max_ctx + max_n) / 64) must stay below 2^31, else GRAFT_EINVAL.
 * lse (device fp32 [rows, Hq], natural log) may be NULL.
 * d in {64, 128}; Hq % Hkv == 0; Hq / Hkv <= 16.
 * ws (device, 16-byte aligned) holds the split partials and the requests'
 *   chunk offsets: at least graft_tree_attention_workspace_bytes(...) bytes
 *   (> 0 for B > 0; its contents need no clearing).
 * Output is bf16 rounded to nearest even; softmax and accumulation fp32.
 * The key ranges are dealt over the workgroups by the batch's total work,
 * so where a request's keys are split (and so its rounding) depends on the
 * whole batch; a call is deterministic for given inputs.
 */
size_t graft_tree_attention_workspace_bytes(int B, int Hq, int Hkv, int d, int max_ctx, int max_n);
int graft_tree_attention(int B, int Hq, int Hkv, int d, float scale,
                         const graft_bf16 *q, const graft_bf16 *kcache, const graft_bf16 *vcache,
                         const int64_t *kv_off, int64_t kv_head_stride,
                         const int32_t *ctx_len, int max_ctx, const int32_t *n, int max_n,
                         const int32_t *row_off, const uint64_t *mask,
                         graft_bf16 *out, float *lse, void *ws, size_t ws_bytes,
                         int32_t *err_flag, graft_stream stream);

/*
 * lm-head and vocabulary top-k (Graft page, section 2: the verification
 * pass yields each position's next-token distribution; the table keeps
 * each token's top successors; greedy acceptance reads the argmax).
 *
 *   logits[m, v] = sum_h hidden[m, h] * W[v, h]     (fp32 accumulate)
 *   topk_id[m, :] = the k ids of row m by (logit desc, id asc), topk_val
 *   the matching logits; argmax = topk_id[m, 0].
 * hidden (device bf16 [M, H]); w (device) holds W in layout w_layout:
 *   GRAFT_W_ROWMAJOR  bf16 [V, H] row-major, H % 64 == 0;
 *   GRAFT_W_PACKED    the output of graft_lmhead_pack, H % 128 == 0,
 *                     M <= 16384 (the faster path: linear weight reads).
 * logits (device fp32 [M, V]), topk_id (device int32 [M, k]),
 * topk_val (device fp32 [M, k], may be NULL).
 * Modes:  hidden && logits && k == 0      -> logits only
 *         !hidden && logits && k > 0      -> top-k of the given logits
 *         hidden && logits && k > 0       -> both, logits materialised
 *         hidden && !logits && k > 0      -> fused: per-row top-k of the
 *                                            logits, which never reach
 *                                            memory (the serving mode)
 * The logits, and so the top-k, are bit-identical for both layouts and
 * all modes.  1 <= k <= min(GRAFT_MAX_K, V) when k is used; V <= GRAFT_MAX_V.
 * ws (device): graft_lmhead_topk_workspace_bytes(M, V, k) bytes (enough
 * for every mode and layout).
 */
#define GRAFT_W_ROWMAJOR 0
#define GRAFT_W_PACKED 1
size_t graft_lmhead_topk_workspace_bytes(int M, int V, int k);
int graft_lmhead_topk(int M, int H, int V, int k,
                      const graft_bf16 *hidden, const graft_bf16 *w, int w_layout, float *logits,
                      int32_t *topk_id, float *topk_val, void *ws, size_t ws_bytes,
                      graft_stream stream);

/*
 * graft_lmhead_topk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the fused packed mode (hidden given,
 * logits not materialised, w_packed from graft_lmhead_pack, H % 128 == 0,
 * 1 <= k <= min(GRAFT_MAX_K, V), V <= GRAFT_MAX_V)
 * with its scratch (the per-(row, workgroup) candidate lists) in an array
 * built into the library, GRAFT_NOALLOC_SCRATCH_BYTES per GPU, held until the
 * process ends.  graft_lmhead_topk_noalloc_bytes(M, k) is the scratch a call
 * needs (at most 8 MiB for M <= 16384 and k <= 16 with the current tilings;
 * 960 rows at k = 8 need 3.75 MiB); a call that needs more returns
 * GRAFT_EINVAL.  Results equal graft_lmhead_topk's bit for bit.  The call
 * allocates nothing; calls that overlap on one GPU share its array and race.
 */
#define GRAFT_NOALLOC_SCRATCH_BYTES (8u << 20)
size_t graft_lmhead_topk_noalloc_bytes(int M, int k);
int graft_lmhead_topk_noalloc(int M, int H, int V, int k, const graft_bf16 *hidden, const graft_bf16 *w_packed,
                              int32_t *topk_id, float *topk_val, graft_stream stream);

/*
 * Weight packing for graft_lmhead_topk (done once, when the lm-head is
 * loaded; not part of a round).  w (device bf16 [V, H] row-major) is
 * rewritten into w_packed (device, graft_lmhead_pack_bytes(V, H) bytes,
 * caller-owned): images of 128 vocabulary rows x 64 hidden columns
 * (row-major inside, 16 KB) in tile-major, column-chunk-minor order, rows
 * past V zero.  H % 128 == 0; returns 0 bytes / GRAFT_EINVAL otherwise.
 */
size_t graft_lmhead_pack_bytes(int V, int H);
int graft_lmhead_pack(int V, int H, const graft_bf16 *w, graft_bf16 *w_packed, graft_stream stream);

/*
 * Greedy acceptance (Graft page, section 2, third step: draft and
 * retrieved nodes face the same rule; TreeGraft page, sections 1 and 5:
 * temperature 0, the accepted prefix stops at the first rejection).
 * Node i > 0 is accepted iff token[i] == argmax[parent[i]] and its parent
 * is accepted (argmax[r] = topk_id[r * k]); the root is accepted.
 * Per request: best = the deepest accepted node (ties: lowest index),
 *   acc_len[b] = depth(best) (draft tokens accepted, bonus excluded),
 *   acc_path[b * 64 + t] = node index at depth t of best's root path for
 *   t <= depth(best), -1 after it; bonus[b] = argmax[best].
 * n, row_off, parent, token, topk_id: device, padded row layout.
 * Outputs: device int32.  Malformed trees flag ERR_PARENT / ERR_CAPACITY
 * and return acc_len 0, path [0], bonus argmax[0] (or -1 if n < 1).
 */
int graft_accept(int B, const int32_t *n, const int32_t *row_off,
                 const int32_t *parent, const int32_t *token, const int32_t *topk_id, int k,
                 int32_t *acc_len, int32_t *acc_path, int32_t *bonus, int32_t *err_flag,
                 graft_stream stream);

/*
 * Sampling at temperature T > 0.  Verification by rejection sampling keeps
 * the target's output distribution (TreeGraft page, section 3 and its
 * reading list); the pages evaluate at T = 1 as well as T = 0 (Graft page,
 * section 5) but give no rule for a node with several children.  This
 * library's reading, lossless for a draft tree whose tokens are chosen:
 * every node draws y ~ softmax(logits / T); the path moves to the
 * lowest-index child whose token is the parent's draw and stops at the first
 * node where none is; that draw is the bonus token.
 *
 * Draws use the Gumbel-max identity with the noise as an input:
 *   y[r] = argmax_t s(r, t),  s(r, t) = fl(fl(l(r, t) * fl(1/T)) + g[r * V + t])
 * (two fp32 operations, each rounded to nearest; ties to the lower t; a
 * NaN score ranks below every number).  g (device fp32 [M, V]) holds
 * i.i.d. Gumbel(0, 1) noise, fresh for every round.  temperature: positive
 * and finite (T = 0 is graft_lmhead_topk + graft_accept).
 *
 * graft_lmhead_topk_sample: the fused, packed lm-head of graft_lmhead_topk
 * (w_packed from graft_lmhead_pack, H % 128 == 0, M <= 16384) producing in
 * the same pass over W the top-k (topk_id, topk_val as graft_lmhead_topk:
 * the successor table still takes the target's top-k) and sample_id
 * (device int32 [M]).  ws: graft_lmhead_sample_workspace_bytes(M, V, k).
 * The logits are identical to graft_lmhead_topk's, so the draws equal
 * graft_sample_rows on the logits graft_lmhead_topk materialises.
 *
 * graft_sample_rows: the same draws on materialised logits (device fp32
 * [M, V]).
 *
 * graft_accept_sampled: graft_accept with sample_id (device int32, one per
 * row of the padded layout) in place of the argmax and only the lowest-index
 * matching child accepted; outputs and error handling as graft_accept,
 * bonus[b] = sample_id at the last accepted node.
 */
size_t graft_lmhead_sample_workspace_bytes(int M, int V, int k);
int graft_lmhead_topk_sample(int M, int H, int V, int k, float temperature, const graft_bf16 *hidden,
                             const graft_bf16 *w_packed, const float *gumbel, int32_t *topk_id,
                             float *topk_val, int32_t *sample_id, void *ws, size_t ws_bytes,
                             graft_stream stream);
int graft_sample_rows(int M, int V, float temperature, const float *logits, const float *gumbel,
                      int32_t *sample_id, graft_stream stream);
int graft_accept_sampled(int B, const int32_t *n, const int32_t *row_off, const int32_t *parent,
                         const int32_t *token, const int32_t *sample_id, int32_t *acc_len,
                         int32_t *acc_path, int32_t *bonus, int32_t *err_flag, graft_stream stream);

/*
 * KV compaction and round chaining (Graft page, section 2, third step: the
 * flattened tree is verified in one pass and only the accepted output is
 * kept; the next round drafts from the bonus token).  The tree's K/V sit
 * at slots ctx .. ctx+n-1 in flattened order (the layout graft_tree_attention
 * reads), so after acceptance the cache must hold, after the ctx context
 * tokens, the accepted path root, p1, .., pa in order:
 *   for every layer l < n_layers, KV head h < Hkv and t = 0 .. acc_len[b]:
 *     slot ctx + t  <-  slot ctx + acc_path[b * 64 + t]   (K and V rows)
 *   ctx_next[b]  = ctx_len[b] + acc_len[b] + 1
 *   root_next[b] = bonus[b]
 * Row (b, l, h, s) of kcache / vcache (device bf16, updated in place) starts
 * at element l * layer_stride + kv_off[b] + h * kv_head_stride + s * d.
 * ctx_len, acc_len, acc_path (graft_accept's layout), bonus, n (tree sizes):
 * device int32.  ctx_next, root_next: device int32 [B], which must not alias
 * ctx_len (every workgroup of a request reads it); chained rounds alternate
 * two buffers.  Slots past ctx + acc_len are left as they are.  A request
 * whose path is malformed (acc_len outside [0, 63], acc_path[0] != 0, not
 * increasing, or a node >= n) flags ERR_PARENT, one whose tree does not fit
 * (ctx + n > kv_head_stride / d) flags ERR_CAPACITY; neither moves any row,
 * and both get ctx_next = ctx_len, root_next = -1.
 * d in {64, 128}; n_layers >= 1; layer_stride >= B-wide cache extent when
 * n_layers > 1 (not checked: the caller's layout).
 */
int graft_kv_compact(int B, int Hkv, int d, int n_layers, graft_bf16 *kcache, graft_bf16 *vcache,
                     int64_t layer_stride, const int64_t *kv_off, int64_t kv_head_stride,
                     const int32_t *ctx_len, const int32_t *n, const int32_t *acc_len,
                     const int32_t *acc_path, const int32_t *bonus, int32_t *ctx_next,
                     int32_t *root_next, int32_t *err_flag, graft_stream stream);

/*
 * Host helper: the stage-adaptive retrieval template of R nodes (Graft
 * page, section 2, second step: asymmetric, higher-ranked successors get
 * more children and a deeper main chain; section 5: depth about 8 and
 * width about 8 work best).  The pages give properties, not a node list;
 * this builds the R best rank paths (r1..rd), d <= dmax, 0 <= r < k, by
 * score prod 0.75/(r+1), ties to smaller depth then lexicographically
 * smaller path.  Output in (host) tmpl_parent[R] (-1 = root) and
 * tmpl_rank[R], topologically ordered.  dmax <= 8, k <= GRAFT_MAX_K,
 * R <= GRAFT_MAX_NODES.
 */
int graft_make_template(int R, int k, int dmax, int32_t *tmpl_parent, int32_t *tmpl_rank);

/*
 * Host helper: Graft's stage budgets of 60 verify slots (Graft page,
 * section 2, second step): pruning at checkpoint depth 0 keeps 8 draft
 * nodes and retrieves 52; depth 1 keeps 24 and retrieves 36; depth 5 keeps
 * 40 and retrieves 20; no pruning (stage -1) keeps the 60-node draft tree
 * and retrieves none.  Draft counts include the root.
 */
int graft_stage_budget(int stage, int32_t *draft_nodes, int32_t *retrieved_nodes);

#ifdef __cplusplus
}
#endif

#endif /* GRAFT_H */
