// Cache-aware ordering of the waiting requests (SGLang paper notes, section 3
// cache-aware scheduling and appendix A.2; vLLM-vs-SGLang page, cache-aware
// ordering): instead of arrival order, run next the request whose prompt
// shares the longest prefix with what will be cached when it runs -- the
// radix tree now, plus the requests already placed ahead of it in this
// round.  Greedy, one placement at a time; ties to the earliest arrival;
// shared lengths in whole matching units; more than fcfs_above waiting:
// arrival order.
//
// Cost.  The shared prefix of two prompts is read off their lexicographic
// order: sort the prompts once, take the common prefix of each sorted
// neighbour pair, and the common prefix of any two prompts is the minimum of
// those neighbour values between them.  One placement then updates every
// candidate with a walk outwards from the placed prompt's sorted position,
// carrying that running minimum: O(n) per placement, O(n^2 + n log n * L)
// for the round instead of comparing prompts pairwise after every placement.
#include <algorithm>
#include <numeric>
#include <vector>

#include "common.h"
#include "radix_tree.h"

using rdx::fail;

extern "C" int rdx_schedule(const rdx_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* offsets,
                            int32_t fcfs_above, int32_t* out_order, int64_t* out_score) {
  if (!t || num_reqs < 0 || fcfs_above < 0) return fail(RDX_EINVAL, "rdx_schedule: bad arguments");
  if (num_reqs == 0) return rdx::ok();
  if (!tokens || !offsets || !out_order || !out_score) return fail(RDX_EINVAL, "rdx_schedule: null array");
  const int32_t n = num_reqs;
  for (int32_t i = 0; i < n; ++i)
    if (offsets[i + 1] < offsets[i])
      return fail(RDX_EINVAL, "rdx_schedule: offsets decrease at request %d", i);
  if (n > fcfs_above) {
    for (int32_t i = 0; i < n; ++i) {
      out_order[i] = i;
      out_score[i] = 0;
    }
    return rdx::ok();
  }
  const rdx::RadixTree& tr = t->impl;
  const int64_t unit = tr.match_unit();
  auto seq = [&](int32_t i) { return tokens + offsets[i]; };
  auto len = [&](int32_t i) { return offsets[i + 1] - offsets[i]; };

  std::vector<int64_t> best(n);
  for (int32_t i = 0; i < n; ++i) best[i] = tr.peek_match(seq(i), len(i));

  // lexicographic order of the prompts, pos[i] = place of request i in it,
  // adj[p] = common prefix of sorted neighbours p-1 and p
  std::vector<int32_t> sorted(n), pos(n);
  std::iota(sorted.begin(), sorted.end(), 0);
  auto shared = [&](int32_t a, int32_t b) { return rdx::common_prefix(seq(a), seq(b), std::min(len(a), len(b))); };
  std::sort(sorted.begin(), sorted.end(), [&](int32_t a, int32_t b) {
    const int64_t c = shared(a, b);
    return c == len(a) ? c < len(b) : (c < len(b) && seq(a)[c] < seq(b)[c]);
  });
  std::vector<int64_t> adj(n, 0);
  for (int32_t p = 0; p < n; ++p) {
    pos[sorted[p]] = p;
    if (p > 0) adj[p] = shared(sorted[p - 1], sorted[p]);
  }

  std::vector<char> placed(n, 0);
  for (int32_t k = 0; k < n; ++k) {
    int32_t pick = -1;
    for (int32_t i = 0; i < n; ++i)
      if (!placed[i] && (pick < 0 || best[i] > best[pick])) pick = i;
    placed[pick] = 1;
    out_order[k] = pick;
    out_score[k] = best[pick];
    // every request still waiting can reuse the placed prompt's prefix
    const int32_t p0 = pos[pick];
    int64_t run = len(pick);
    for (int32_t p = p0 + 1; p < n && run > 0; ++p) {
      run = std::min(run, adj[p]);
      const int32_t j = sorted[p];
      if (!placed[j]) best[j] = std::max(best[j], (run / unit) * unit);
    }
    run = len(pick);
    for (int32_t p = p0 - 1; p >= 0 && run > 0; --p) {
      run = std::min(run, adj[p + 1]);
      const int32_t j = sorted[p];
      if (!placed[j]) best[j] = std::max(best[j], (run / unit) * unit);
    }
  }
  return rdx::ok();
}
