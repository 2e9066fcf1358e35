"""Oracle: a plain, slow CPU statement of one round of tree speculative
decoding, used as TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline
leg may import or run anything in this package.  The GPU library never
links, imports or falls back to it, and this package shares no code with
the GPU path (it imports nothing from it).

Sources (three web pages on the method):
  * Graft page -- write-up of arXiv:2605.20104 (Zhejiang U. / Alibaba Qwen /
    USTC): pruning at checkpoints, retrieval from a GPU successor table with
    a stage-adaptive template, flatten + tree positions + mask, one parallel
    verification, online table update.
  * TreeGraft page -- reading notes on arXiv:2608.26112: EAGLE-style tree
    construction with cumulative scores and a global prune to Bver, tree
    attention verification.
  * BlockPilot page -- write-up of arXiv:2606.31315: the prefix-survival
    view of the accepted length.

Floating point is fp64 (inputs given in bf16/fp32 are upcast exactly),
except where a float decides an integer: candidate scores and logits are
ranked in the fp32 they are given in, as the GPU path does.

Modules:
  tree       -- draft selection, retrieved-node append, static replacement,
                flatten, depth / positions / ancestor mask
  template   -- the stage-adaptive retrieval template (a proposed rule; the
                pages fix only its properties -- parity unpinned in shape)
  table      -- successor-table update and template retrieval
  attention  -- tree-masked GQA attention
  lmhead     -- logits = hidden . W^T
  topk       -- per-row top-k / argmax, ties to the lower id
  accept     -- greedy acceptance: deepest accepted node, path, bonus token
  sample     -- acceptance at temperature T > 0: Gumbel-max draws per node,
                first matching child (a reading: the pages give no rule)
  treegraft  -- TreeGraft's shared tree from a small and a mid drafter
                (extended pool, non-destructive graft) before the prune
  tail       -- Graft-TAIL: a block draft's confident prefix kept, its tail
                replaced by retrieval under the deepest kept node
  kv         -- KV compaction to the accepted path and round chaining
  round      -- the above composed into one round
"""


class OracleError(ValueError):
    """An input the method does not define (e.g. a token outside [0, V))."""
