// Internal launch helpers shared between the C-ABI translation units.
#pragma once

#include "common.h"

namespace graft {

struct TopkPlan {
  int slices;
  int slice_len;
  size_t ws_bytes;
};

// Vocabulary split used by the top-k passes (and its workspace size).
TopkPlan topk_plan(int M, int V, int k);
int launch_topk(int M, int V, int k, const float *logits, int32_t *topk_id, float *topk_val, void *ws,
                hipStream_t stream);
// Merges `slices` sorted candidate lists of k (value, id) pairs per row.
int launch_topk_merge(int M, int slices, int k, const uint64_t *part, int32_t *topk_id, float *topk_val,
                      hipStream_t stream);
size_t lmhead_fused_ws_bytes(int M, int V, int k);

}  // namespace graft
