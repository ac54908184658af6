// Throughput-oriented token batching (BatchLLM explainer: Throughput-oriented
// Token Batching with Equations 3-4, three-queue fetching, Memory-centric
// Token Batching).  Requests sharing a prefix form a group; groups run in
// descending decoding ratio R_group = 1 / (prefix + sum of distinct prompts).
// Every iteration takes one decode token from each decoding request, then
// prefill chunks of at most s_chunk tokens -- distinct prompts of groups whose
// prefix is done first, then prefixes -- until the next chunk would take the
// KV memory (2 entries per token: the decoding groups' prefixes once, the
// decoding requests' own tokens, the chunks taken) above the threshold.
//
// State is kept in queue order so an iteration costs O(entries it emits):
// the decoding list, the distinct-prompt queue and the prefix queue are
// vectors sorted by (group rank, member index); members and groups that
// become ready during an iteration are merged in at its end (they are served
// from the next iteration on).
#include <algorithm>
#include <new>
#include <numeric>
#include <vector>

#include "common.h"

struct rdx_batcher {
  int32_t num_groups = 0, s_chunk = 0;
  int64_t threshold = 0;
  std::vector<int32_t> prefix_len, member_off, distinct_len, decode_len, group_of;
  std::vector<int32_t> rank;       // group -> position in the group order
  std::vector<int32_t> pre_done;   // per group
  std::vector<int32_t> dist_done;  // per member
  std::vector<int32_t> generated;  // per member
  // queues, each sorted by (rank of group, member index)
  std::vector<int32_t> decoding;   // members
  std::vector<int32_t> distinct_q; // members whose group prefix is done and prompt is not
  std::vector<int32_t> prefix_q;   // groups, by rank
  std::vector<int32_t> new_dec, new_dist, tmp;
  int64_t iteration = 0;

  int64_t key(int32_t m) const { return ((int64_t)rank[group_of[m]] << 32) | (m - member_off[group_of[m]]); }
  void merge_into(std::vector<int32_t>& q, std::vector<int32_t>& add) {
    if (add.empty()) return;
    auto less = [&](int32_t a, int32_t b) { return key(a) < key(b); };
    std::sort(add.begin(), add.end(), less);
    tmp.resize(q.size() + add.size());
    std::merge(q.begin(), q.end(), add.begin(), add.end(), tmp.begin(), less);
    q.swap(tmp);
    add.clear();
  }
};

using rdx::fail;

extern "C" {

int rdx_batcher_create(int32_t num_groups, const int32_t* prefix_len, const int32_t* member_offsets,
                       const int32_t* distinct_len, const int32_t* decode_len, int32_t s_chunk, int64_t m_threshold,
                       rdx_batcher** out) {
  if (!out || num_groups < 0 || !prefix_len || !member_offsets || s_chunk < 1 || m_threshold < 2 * (int64_t)s_chunk)
    return fail(RDX_EINVAL, "rdx_batcher_create: bad arguments (need s_chunk >= 1, m_threshold >= 2 s_chunk)");
  if (member_offsets[0] != 0) return fail(RDX_EINVAL, "rdx_batcher_create: member_offsets[0] must be 0");
  for (int32_t g = 0; g < num_groups; ++g) {
    if (member_offsets[g + 1] <= member_offsets[g])
      return fail(RDX_EINVAL, "rdx_batcher_create: group %d has no members", g);
    if (prefix_len[g] < 0) return fail(RDX_EINVAL, "rdx_batcher_create: group %d: negative prefix", g);
  }
  const int32_t nm = member_offsets[num_groups];
  if (nm > 0 && (!distinct_len || !decode_len)) return fail(RDX_EINVAL, "rdx_batcher_create: null member array");
  for (int32_t m = 0; m < nm; ++m)
    if (distinct_len[m] < 1 || decode_len[m] < 0)
      return fail(RDX_EINVAL, "rdx_batcher_create: member %d: need distinct >= 1 and decode >= 0", m);
  rdx_batcher* b;
  try {
    b = new rdx_batcher();
    b->num_groups = num_groups;
    b->s_chunk = s_chunk;
    b->threshold = m_threshold;
    b->prefix_len.assign(prefix_len, prefix_len + num_groups);
    b->member_off.assign(member_offsets, member_offsets + num_groups + 1);
    b->distinct_len.assign(distinct_len, distinct_len + nm);
    b->decode_len.assign(decode_len, decode_len + nm);
    b->group_of.resize(nm);
    std::vector<int64_t> prefill(num_groups, 0);
    for (int32_t g = 0; g < num_groups; ++g) {
      prefill[g] = prefix_len[g];
      for (int32_t m = member_offsets[g]; m < member_offsets[g + 1]; ++m) {
        b->group_of[m] = g;
        prefill[g] += distinct_len[m];
      }
    }
    // descending 1 / prefill = ascending prefill tokens, ties by index
    std::vector<int32_t> order(num_groups);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t c) { return prefill[a] < prefill[c]; });
    b->rank.resize(num_groups);
    for (int32_t r = 0; r < num_groups; ++r) b->rank[order[r]] = r;
    b->pre_done.assign(num_groups, 0);
    b->dist_done.assign(nm, 0);
    b->generated.assign(nm, 0);
    for (int32_t g : order) {
      if (prefix_len[g] > 0)
        b->prefix_q.push_back(g);
      else
        for (int32_t m = member_offsets[g]; m < member_offsets[g + 1]; ++m) b->distinct_q.push_back(m);
    }
  } catch (const std::bad_alloc&) {
    return fail(RDX_EINVAL, "rdx_batcher_create: out of host memory");
  }
  *out = b;
  return rdx::ok();
}

void rdx_batcher_destroy(rdx_batcher* b) { delete b; }

int rdx_batcher_next(rdx_batcher* b, rdx_tb_entry* out, int32_t cap, int32_t* out_n) {
  if (!b || !out_n || cap < 0 || (cap > 0 && !out)) return fail(RDX_EINVAL, "rdx_batcher_next: bad arguments");
  *out_n = 0;
  // pass 1: how many entries (nothing changes yet)
  const int64_t nd = (int64_t)b->decoding.size();
  int64_t memory = 0;
  // a group's prefix once (decoding is sorted by group), each request's own tokens
  for (int64_t i = 0; i < nd; ++i) {
    const int32_t m = b->decoding[i], g = b->group_of[m];
    if (i == 0 || b->group_of[b->decoding[i - 1]] != g) memory += 2 * (int64_t)b->prefix_len[g];
    memory += 2 * ((int64_t)b->distinct_len[m] + b->generated[m]);
  }
  // The batch is bounded by KV memory (BatchLLM explainer, Memory-centric
  // Token Batching): beside what the decoding requests hold, the iteration
  // takes prefill chunks from the head of the queue -- distinct prompts,
  // then prefixes -- as long as their K/V entries fit under the threshold.
  const int64_t n2 = (int64_t)b->distinct_q.size(), n3 = (int64_t)b->prefix_q.size();
  auto remaining = [&](int64_t i) -> int64_t {
    if (i < n2) return b->distinct_len[b->distinct_q[i]] - b->dist_done[b->distinct_q[i]];
    const int32_t g = b->prefix_q[i - n2];
    return b->prefix_len[g] - b->pre_done[g];
  };
  int64_t budget = b->threshold - memory;  // K/V entries left for chunks
  int64_t n_chunks = 0;
  for (; n_chunks < n2 + n3; ++n_chunks) {
    budget -= 2 * std::min<int64_t>(b->s_chunk, remaining(n_chunks));
    if (budget < 0) break;
  }
  const int64_t total = nd + n_chunks;
  if (total == 0) return rdx::ok();  // the job is done
  if (total > cap) {
    *out_n = (int32_t)total;
    return fail(RDX_ENOBUFS, "rdx_batcher_next: %lld entries, capacity %d", (long long)total, cap);
  }
  // pass 2: emit and advance
  int32_t k = 0;
  for (int32_t m : b->decoding) {
    const int32_t g = b->group_of[m];
    out[k++] = {RDX_TB_DECODE, g, m, b->prefix_len[g] + b->distinct_len[m] + b->generated[m], 1};
    b->generated[m]++;
  }
  int64_t taken2 = 0, taken3 = 0;
  for (int64_t i = 0; i < n_chunks; ++i) {
    if (i < n2) {
      const int32_t m = b->distinct_q[i];
      const int32_t g = b->group_of[m];
      const int32_t c = std::min(b->s_chunk, b->distinct_len[m] - b->dist_done[m]);
      out[k++] = {RDX_TB_DISTINCT, g, m, b->prefix_len[g] + b->dist_done[m], c};
      b->dist_done[m] += c;
      if (b->dist_done[m] == b->distinct_len[m] && b->decode_len[m] > 0) b->new_dec.push_back(m);
      ++taken2;
    } else {
      const int32_t g = b->prefix_q[i - n2];
      const int32_t c = std::min(b->s_chunk, b->prefix_len[g] - b->pre_done[g]);
      out[k++] = {RDX_TB_PREFIX, g, -1, b->pre_done[g], c};
      b->pre_done[g] += c;
      if (b->pre_done[g] == b->prefix_len[g])
        for (int32_t m = b->member_off[g]; m < b->member_off[g + 1]; ++m) b->new_dist.push_back(m);
      ++taken3;
    }
  }
  // drop what finished, merge in what became ready (served next iteration)
  auto& dq = b->decoding;
  dq.erase(std::remove_if(dq.begin(), dq.end(), [&](int32_t m) { return b->generated[m] == b->decode_len[m]; }),
           dq.end());
  auto& q2 = b->distinct_q;
  q2.erase(std::remove_if(q2.begin(), q2.begin() + taken2,
                          [&](int32_t m) { return b->dist_done[m] == b->distinct_len[m]; }),
           q2.begin() + taken2);
  auto& q3 = b->prefix_q;
  q3.erase(std::remove_if(q3.begin(), q3.begin() + taken3,
                          [&](int32_t g) { return b->pre_done[g] == b->prefix_len[g]; }),
           q3.begin() + taken3);
  b->merge_into(dq, b->new_dec);
  b->merge_into(q2, b->new_dist);
  b->iteration++;
  *out_n = k;
  return rdx::ok();
}

}  // extern "C"
