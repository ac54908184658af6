// Global prefix analysis (BatchLLM explainer, Global Prefix Sharing): the
// requests of a batch form one radix tree; a dynamic program decides where
// the leaves below a node keep one group (one shared prefix, computed once;
// each member computes the rest of its prompt) and where they split into
// groups further down -- the explainer's gain-versus-penalty test applied at
// every node.  The result minimises the processed prefill tokens
//   sum of group prefixes + sum of (prompt - its group's prefix),
// the N_processed of the token-saving ratio (Equation 2).
//
// The tree is never materialised token by token.  Sorting the prompts puts
// every subtree in a contiguous range whose shared depth is the minimum of
// the neighbour common prefixes inside it; a node is such a range, its
// children the sub-ranges cut where that minimum is reached, and the
// requests whose prompt ends at the node's depth sort first in it.  Along an
// unbranched edge the DP never prefers an inner token node when two or more
// requests share it (one group deeper saves tokens), and for a lone request
// every node of its edge costs the same; ties keep the higher node, so a
// lone request is grouped at the first token of its own edge.
#include <algorithm>
#include <numeric>
#include <vector>

#include "common.h"
#include "radix_tree.h"

namespace {

struct Range {
  int32_t lo, hi;      // sorted positions [lo, hi)
  int64_t depth;       // shared depth of the range (a node), or the parent's
  int32_t parent_node; // for the assignment pass
};

}  // namespace

using rdx::fail;

extern "C" int rdx_prefix_groups(int32_t num_reqs, const int32_t* tokens, const int64_t* offsets,
                                 int32_t* out_group, int64_t* out_prefix, int32_t* out_num_groups,
                                 int64_t* out_processed) {
  if (num_reqs < 0 || !out_num_groups || !out_processed) return fail(RDX_EINVAL, "rdx_prefix_groups: bad arguments");
  *out_num_groups = 0;
  *out_processed = 0;
  if (num_reqs == 0) return rdx::ok();
  if (!tokens || !offsets || !out_group || !out_prefix) return fail(RDX_EINVAL, "rdx_prefix_groups: null array");
  const int32_t n = num_reqs;
  for (int32_t i = 0; i < n; ++i)
    if (offsets[i + 1] < offsets[i]) return fail(RDX_EINVAL, "rdx_prefix_groups: offsets decrease at %d", i);
  auto seq = [&](int32_t i) { return tokens + offsets[i]; };
  auto len = [&](int32_t i) { return offsets[i + 1] - offsets[i]; };
  auto shared = [&](int32_t a, int32_t b) { return rdx::common_prefix(seq(a), seq(b), std::min(len(a), len(b))); };

  std::vector<int32_t> sorted(n);
  std::iota(sorted.begin(), sorted.end(), 0);
  std::stable_sort(sorted.begin(), sorted.end(), [&](int32_t a, int32_t b) {
    const int64_t c = shared(a, b);
    return c == len(a) ? c < len(b) : (c < len(b) && seq(a)[c] < seq(b)[c]);
  });
  std::vector<int64_t> adj(n, 0), pre_len(n + 1, 0);
  for (int32_t p = 0; p < n; ++p) {
    if (p > 0) adj[p] = shared(sorted[p - 1], sorted[p]);
    pre_len[p + 1] = pre_len[p] + len(sorted[p]);
  }

  // ---- nodes, top-down: a node = a sorted range with >= 2 requests ----
  struct Node {
    int32_t lo, hi, n_end;   // n_end: requests ending at this depth (first in the range)
    int64_t depth;
    std::vector<int32_t> kids;   // child nodes
    std::vector<int32_t> leaves; // sorted positions of lone requests below
    int64_t cost = 0;
    bool here = false;
  };
  std::vector<Node> nodes;
  if (n == 1) {
    // one request: the root keeps it (ties keep the higher node)
    out_group[0] = 0;
    out_prefix[0] = 0;
    *out_num_groups = 1;
    *out_processed = len(0);
    return rdx::ok();
  }
  {
    std::vector<std::pair<int32_t, int32_t>> todo;  // (range lo, hi) with parent node index
    std::vector<int32_t> todo_parent;
    todo.push_back({0, n});
    todo_parent.push_back(-1);
    while (!todo.empty()) {
      auto [lo, hi] = todo.back();
      const int32_t par = todo_parent.back();
      todo.pop_back();
      todo_parent.pop_back();
      int64_t d = INT64_MAX;
      for (int32_t p = lo + 1; p < hi; ++p) d = std::min(d, adj[p]);
      const int32_t id = (int32_t)nodes.size();
      nodes.push_back(Node{lo, hi, 0, d, {}, {}});
      if (par >= 0) nodes[par].kids.push_back(id);
      int32_t p = lo;
      while (p < hi && len(sorted[p]) == d) ++p;
      nodes[id].n_end = p - lo;
      // children: maximal sub-ranges of [p, hi) whose neighbours share more than d
      while (p < hi) {
        int32_t q = p + 1;
        while (q < hi && adj[q] > d) ++q;
        if (q - p == 1) {
          nodes[id].leaves.push_back(p);
        } else {
          todo.push_back({p, q});
          todo_parent.push_back(id);
        }
        p = q;
      }
    }
  }
  // ---- costs, bottom-up (children have larger indices than parents) ----
  for (int32_t v = (int32_t)nodes.size() - 1; v >= 0; --v) {
    Node& x = nodes[v];
    const int64_t cnt = x.hi - x.lo;
    const int64_t here = x.depth + (pre_len[x.hi] - pre_len[x.lo]) - cnt * x.depth;
    int64_t split = x.n_end > 0 ? x.depth : 0;
    for (int32_t k : x.kids) split += nodes[k].cost;
    for (int32_t p : x.leaves) split += len(sorted[p]);
    x.here = here <= split;
    x.cost = std::min(here, split);
  }
  // the root: the top range when it branches at depth 0; when every request
  // shares d > 0 tokens the root and the edge above the range lose strictly
  *out_processed = nodes[0].cost;
  // ---- assignment, top-down ----
  std::vector<int32_t> gnode(n, -1);   // group key per request
  std::vector<int64_t> gdepth(n, 0);
  int32_t key = 0;
  std::vector<int32_t> stack{0};
  while (!stack.empty()) {
    const int32_t v = stack.back();
    stack.pop_back();
    const Node& x = nodes[v];
    if (x.here) {
      for (int32_t p = x.lo; p < x.hi; ++p) {
        gnode[sorted[p]] = key;
        gdepth[sorted[p]] = x.depth;
      }
      ++key;
      continue;
    }
    if (x.n_end > 0) {
      for (int32_t p = x.lo; p < x.lo + x.n_end; ++p) {
        gnode[sorted[p]] = key;
        gdepth[sorted[p]] = x.depth;
      }
      ++key;
    }
    for (int32_t p : x.leaves) {
      gnode[sorted[p]] = key++;
      gdepth[sorted[p]] = x.depth + 1;
    }
    for (int32_t k : x.kids) stack.push_back(k);
  }
  // group ids in order of their first request
  std::vector<int32_t> remap(key, -1);
  int32_t ng = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t& g = remap[gnode[i]];
    if (g < 0) g = ng++;
    out_group[i] = g;
    out_prefix[i] = gdepth[i];
  }
  *out_num_groups = ng;
  return rdx::ok();
}
