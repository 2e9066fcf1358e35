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

}  // namespace graft
