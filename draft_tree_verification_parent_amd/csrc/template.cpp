// Host helpers: the stage-adaptive retrieval template and Graft's stage
// budgets (Graft page, arXiv:2605.20104 write-up, section 2, second step;
// section 5 for the depth-8 / width-8 optimum).
//
// The pages describe the template only by its properties (asymmetric: higher
// ranked successors get more children and a deeper main chain; lower ranks
// keep width).  The rule built here: the R best rank paths (r1..rd),
// d <= dmax, 0 <= r < k, scored prod 0.75/(r+1), ties to the smaller depth
// and then the lexicographically smaller path.  Selection grows the template
// one node at a time from a frontier of candidate children, comparing
// scores exactly in integers:
//   score(a) > score(b)  <=>  3^da * 4^db * Pb  >  3^db * 4^da * Pa,
// with P = prod (r+1) (fits in 128 bits for dmax <= 8, k <= 16).
#include <cstring>
#include <vector>

#include "common.h"

namespace {

struct Cand {
  int depth;
  unsigned long long prod;  // prod (r+1) over the path
  int path[8];
  int parent;  // template index of the parent path, -1 for the root
};

unsigned __int128 pow_u(unsigned base, int e) {
  unsigned __int128 r = 1;
  for (int i = 0; i < e; ++i) r *= base;
  return r;
}

// true iff a precedes b in template order
bool precedes(const Cand &a, const Cand &b) {
  const unsigned __int128 lhs = pow_u(3, a.depth) * pow_u(4, b.depth) * b.prod;
  const unsigned __int128 rhs = pow_u(3, b.depth) * pow_u(4, a.depth) * a.prod;
  if (lhs != rhs) return lhs > rhs;
  if (a.depth != b.depth) return a.depth < b.depth;
  for (int i = 0; i < a.depth; ++i)
    if (a.path[i] != b.path[i]) return a.path[i] < b.path[i];
  return false;
}

}  // namespace

extern "C" int graft_make_template(int R, int k, int dmax, int32_t *tmpl_parent, int32_t *tmpl_rank) {
  using graft::fail;
  if (R < 0 || R > GRAFT_MAX_NODES || k < 1 || k > GRAFT_MAX_K || dmax < 1 || dmax > 8)
    return fail(GRAFT_EINVAL, "make_template: R=%d k=%d dmax=%d", R, k, dmax);
  if (R > 0 && (!tmpl_parent || !tmpl_rank)) return fail(GRAFT_EINVAL, "make_template: NULL output");
  std::vector<Cand> frontier;
  for (int r = 0; r < k; ++r) {
    Cand c{};
    c.depth = 1;
    c.prod = static_cast<unsigned long long>(r + 1);
    c.path[0] = r;
    c.parent = -1;
    frontier.push_back(c);
  }
  for (int t = 0; t < R; ++t) {
    if (frontier.empty()) return fail(GRAFT_EINVAL, "make_template: R=%d exceeds the k-ary tree of depth %d", R, dmax);
    size_t best = 0;
    for (size_t i = 1; i < frontier.size(); ++i)
      if (precedes(frontier[i], frontier[best])) best = i;
    const Cand chosen = frontier[best];
    frontier.erase(frontier.begin() + static_cast<long>(best));
    tmpl_parent[t] = chosen.parent;
    tmpl_rank[t] = chosen.path[chosen.depth - 1];
    if (chosen.depth < dmax) {
      for (int r = 0; r < k; ++r) {
        Cand c = chosen;
        c.path[c.depth] = r;
        c.depth += 1;
        c.prod *= static_cast<unsigned long long>(r + 1);
        c.parent = t;
        frontier.push_back(c);
      }
    }
  }
  return GRAFT_OK;
}

extern "C" int graft_stage_budget(int stage, int32_t *draft_nodes, int32_t *retrieved_nodes) {
  int d, r;
  switch (stage) {
    case -1: d = 60; r = 0; break;
    case 0: d = 8; r = 52; break;
    case 1: d = 24; r = 36; break;
    case 5: d = 40; r = 20; break;
    default: return graft::fail(GRAFT_EINVAL, "stage_budget: checkpoint depth %d (expected -1, 0, 1, 5)", stage);
  }
  if (draft_nodes) *draft_nodes = d;
  if (retrieved_nodes) *retrieved_nodes = r;
  return GRAFT_OK;
}
