// Batch planner (see plan.h).
//
// Sharing structure.  A tree node reached by two or more requests of the
// batch is shared: its keys are attended once for all of those requests'
// query rows (BatchLLM explainer, Horizontal Fusion: the common-prefix part
// of prefix-shared attention).  Consecutive shared nodes reached by the same
// requests form one segment.  Everything after a request's last shared
// segment -- unshared cached nodes, earlier private tokens, its new tokens --
// is its own range, attended causally (key position <= query position).
//
// Tiles.  Requests are ordered depth-first by their segments so every
// segment's requests are contiguous; their new tokens are packed into tiles
// of kTileRows query rows (token x the Hq/Hkv query heads of one KV head).
// An extend tile never mixes requests with different segment lists; a
// decode tile spans one top-level group, so a prefix is streamed once for
// all of its requests' decode tokens.
//
// Items.  When the launch would have too few (tile, KV head) pairs to fill
// the GPU, the key ranges of a tile are cut into chunks run as separate work
// items; each writes a partial softmax state, and a merge pass right after
// combines them by log-sum-exp.
#include "plan.h"

#include <algorithm>
#include <unordered_map>

#include "common.h"

namespace rdx {

namespace {

int64_t align16(int64_t w) { return (w + 15) & ~int64_t(15); }

struct Seg {
  int64_t start, end;  // key positions
  int rep = -1;        // request whose page-table row is read for this segment
};

struct Req {
  int32_t row, kv_len, q_len, written, q_off, depth, shared_len;
  int64_t new_off;
  std::vector<const Node*> path;
  std::vector<int> segs;  // shared segment ids, top-down
};

}  // namespace

int Plan::build(const RadixTree& tree, const rdx_batch& b, int64_t page_ld) {
  built = false;
  if (b.num_reqs < 0 || (b.num_reqs > 0 && (!b.node || !b.row || !b.kv_len || !b.q_len || !b.written)))
    return fail(RDX_EINVAL, "rdx_plan_build: bad batch pointers");
  if (page_ld <= 0 || page_ld > (int64_t)1 << 30) return fail(RDX_EINVAL, "rdx_plan_build: bad page-table stride");
  const int R = b.num_reqs;
  std::vector<Req> rq(R);
  int64_t total_new = 0;
  std::unordered_map<int32_t, int> row_seen;
  max_page_row = -1;
  for (int r = 0; r < R; ++r) {
    Req& q = rq[r];
    q.row = b.row[r];
    q.kv_len = b.kv_len[r];
    q.q_len = b.q_len[r];
    q.written = b.written[r];
    q.q_off = (int32_t)total_new;
    q.new_off = total_new;
    const Node* n = tree.find(b.node[r]);
    if (!n) return fail(RDX_ESTATE, "rdx_plan_build: request %d: unknown node %lld", r, (long long)b.node[r]);
    for (const Node* p = n; p != tree.root(); p = p->parent) q.path.push_back(p);
    std::reverse(q.path.begin(), q.path.end());
    q.depth = n == tree.root() ? 0 : (int32_t)n->end();
    const int64_t first_new = (int64_t)q.kv_len - q.q_len;
    if (q.row < 0 || q.q_len < 0 || q.q_len > q.kv_len || q.kv_len > page_ld || q.depth > first_new ||
        q.written < 0 || q.written > first_new || (q.written < first_new && q.depth < first_new))
      return fail(RDX_EINVAL,
                  "rdx_plan_build: request %d inconsistent (row %d kv_len %d q_len %d written %d cached %d)", r,
                  q.row, q.kv_len, q.q_len, q.written, q.depth);
    if (!row_seen.emplace(q.row, r).second)
      return fail(RDX_EINVAL, "rdx_plan_build: requests %d and %d share page-table row %d", row_seen[q.row], r, q.row);
    max_page_row = std::max<int64_t>(max_page_row, q.row);
    total_new += q.q_len;
    if (total_new > ((int64_t)1 << 30)) return fail(RDX_EINVAL, "rdx_plan_build: too many new tokens");
  }
  if (total_new > 0 && !b.new_slots) return fail(RDX_EINVAL, "rdx_plan_build: new_slots missing");
  for (int64_t i = 0; i < total_new; ++i)
    if (b.new_slots[i] < 0 || b.new_slots[i] >= desc.num_slots)
      return fail(RDX_EINVAL, "rdx_plan_build: new slot %d out of range", b.new_slots[i]);

  // ---- sharing: nodes reached by >= 2 requests, grouped into segments ----
  std::unordered_map<const Node*, int> cnt;
  for (auto& q : rq)
    for (const Node* n : q.path) cnt[n]++;
  std::unordered_map<const Node*, int> seg_of_first;
  std::vector<Seg> segs;
  for (auto& q : rq) {
    size_t i = 0;
    while (i < q.path.size() && cnt[q.path[i]] >= 2) {
      size_t j = i;
      while (j + 1 < q.path.size() && cnt[q.path[j + 1]] == cnt[q.path[i]]) ++j;
      auto it = seg_of_first.find(q.path[i]);
      int s;
      if (it == seg_of_first.end()) {
        s = (int)segs.size();
        segs.push_back({q.path[i]->start, q.path[j]->end(), -1});
        seg_of_first.emplace(q.path[i], s);
      } else {
        s = it->second;
      }
      q.segs.push_back(s);
      i = j + 1;
    }
    q.shared_len = q.segs.empty() ? 0 : (int32_t)segs[q.segs.back()].end;
  }
  num_shared_segments = (int64_t)segs.size();

  // ---- depth-first order: lexicographic on segment lists (stable) ----
  std::vector<int> order(R);
  for (int r = 0; r < R; ++r) order[r] = r;
  std::stable_sort(order.begin(), order.end(), [&](int a, int c) { return rq[a].segs < rq[c].segs; });
  for (int r : order)
    for (int s : rq[r].segs)
      if (segs[s].rep < 0) segs[s].rep = r;

  // ---- page-table writes: [written, kv_len) of each row ----
  runs.clear();
  run_slots.clear();
  for (int r = 0; r < R; ++r) {
    const Req& q = rq[r];
    if (q.written >= q.kv_len) continue;
    int64_t src = (int64_t)run_slots.size();
    for (const Node* n : q.path) {
      for (int64_t p = std::max<int64_t>(n->start, q.written); p < n->end(); ++p)
        run_slots.push_back(n->slots[p - n->start]);
    }
    for (int64_t i = std::max<int64_t>(0, (int64_t)q.written - (q.kv_len - q.q_len)); i < q.q_len; ++i)
      run_slots.push_back(b.new_slots[q.new_off + i]);
    int64_t count = (int64_t)run_slots.size() - src;
    if (count != q.kv_len - q.written) return fail(RDX_EINVAL, "rdx_plan_build: request %d: page-table gap", r);
    runs.insert(runs.end(), {q.row, q.written, (int32_t)count, (int32_t)src});
  }
  new_slots.assign(b.new_slots, b.new_slots + total_new);

  // ---- tiles ----
  const int tt = tile_tokens();
  toks.clear();
  tiles.clear();
  struct TileReq { int r, lo, hi; };
  std::vector<std::vector<TileReq>> tile_reqs;
  int64_t cur_key = INT64_MIN;
  for (int r : order) {
    const Req& q = rq[r];
    if (q.q_len == 0) continue;
    int64_t key;
    if (kind == RDX_PLAN_EXTEND)
      key = q.segs.empty() ? -1 - (int64_t)r : q.segs.back();
    else
      key = q.segs.empty() ? -1 : q.segs.front();
    for (int t = 0; t < q.q_len; ++t) {
      int ntile = (int)tile_reqs.size();
      bool fresh = ntile == 0 || key != cur_key || tiles[(ntile - 1) * kTileWords + 1] >= tt;
      if (fresh) {
        tiles.insert(tiles.end(), {(int32_t)(toks.size() / kTokWords), 0, 0, 0, -1, 0, 0, 0});
        tile_reqs.emplace_back();
        cur_key = key;
        ntile++;
      }
      int32_t* tl = &tiles[(ntile - 1) * kTileWords];
      auto& trs = tile_reqs.back();
      int local = tl[1];
      if (trs.empty() || trs.back().r != r) trs.push_back({r, local, local});
      trs.back().hi = local + 1;
      tl[1]++;
      toks.push_back(q.q_off + t);
      toks.push_back(q.kv_len - q.q_len + t);
    }
  }
  const int ntiles = (int)tile_reqs.size();

  // ---- jobs per tile (before splitting) ----
  struct Job { int32_t row, k0, k1, lo, hi, causal; };
  std::vector<std::vector<Job>> tile_jobs(ntiles);
  int64_t total_cost = 0;
  for (int t = 0; t < ntiles; ++t) {
    auto& trs = tile_reqs[t];
    std::vector<int> seen;
    std::vector<Job> shared;
    for (auto& tr : trs) {
      for (int s : rq[tr.r].segs) {
        auto it = std::find(seen.begin(), seen.end(), s);
        if (it == seen.end()) {
          seen.push_back(s);
          shared.push_back({rq[segs[s].rep].row, (int32_t)segs[s].start, (int32_t)segs[s].end, tr.lo, tr.hi, 0});
        } else {
          Job& j = shared[it - seen.begin()];
          j.lo = std::min(j.lo, tr.lo);
          j.hi = std::max(j.hi, tr.hi);
        }
      }
    }
    auto& js = tile_jobs[t];
    js = shared;
    for (auto& tr : trs) {
      const Req& q = rq[tr.r];
      if (q.kv_len > q.shared_len) js.push_back({q.row, q.shared_len, q.kv_len, tr.lo, tr.hi, 1});
    }
    for (auto& j : js) total_cost += j.k1 - j.k0;
  }

  // ---- split into items ----
  const int hkv = desc.num_kv_heads;
  // default launch size the split aims for: extend only splits when fewer
  // than ~one round of workgroups (2 per CU) exists; decode aims for ~2 per
  // CU (measured best: larger chunks amortise the Q load and partial write)
  int64_t target = target_items > 0 ? target_items : 512;
  int64_t chunk = INT64_MAX;
  if ((int64_t)ntiles * hkv < target && total_cost > 0) {
    int64_t per_kvh = std::max<int64_t>(1, target / hkv);
    chunk = (total_cost + per_kvh - 1) / per_kvh;
    chunk = std::max<int64_t>(kKeyBlock, (chunk + kKeyBlock - 1) / kKeyBlock * kKeyBlock);
  }
  jobs.clear();
  contribs.clear();
  items.clear();
  cptr.clear();
  clist.clear();
  mblocks.clear();
  num_split_tiles = 0;
  ws_tokens = 0;
  key_rows = 0;
  struct ItemRec { int32_t tile, jb, je, c; int64_t cost; };
  std::vector<ItemRec> its;
  for (int t = 0; t < ntiles; ++t) {
    int32_t* tl = &tiles[t * kTileWords];
    std::vector<ItemRec> mine;
    int64_t cur = 0;
    for (const Job& j : tile_jobs[t]) {
      for (int64_t a = j.k0; a < j.k1;) {
        int64_t room = chunk - cur;
        if (room <= 0 || mine.empty()) {
          mine.push_back({t, (int32_t)(jobs.size() / kJobWords), (int32_t)(jobs.size() / kJobWords),
                          (int32_t)mine.size(), 0});
          cur = 0;
          room = chunk;
        }
        int64_t e = room >= (int64_t)j.k1 - a ? (int64_t)j.k1 : a + room;
        jobs.insert(jobs.end(), {j.row, (int32_t)a, (int32_t)e, j.lo, j.hi, j.causal, 0, 0});
        mine.back().je++;
        mine.back().cost += e - a;
        cur += e - a;
        a = e;
      }
    }
    tl[2] = (int32_t)mine.size();
    tl[3] = (int32_t)(contribs.size() / kContribWords);
    if (mine.size() > 1) {
      tl[4] = (int32_t)num_split_tiles++;
      const int cbase = (int)(contribs.size() / kContribWords);
      for (auto& it : mine) {
        int32_t lo = INT32_MAX, hi = 0;
        for (int32_t jj = it.jb; jj < it.je; ++jj) {
          lo = std::min(lo, jobs[jj * kJobWords + 3]);
          hi = std::max(hi, jobs[jj * kJobWords + 4]);
        }
        contribs.insert(contribs.end(), {lo, hi, (int32_t)ws_tokens, 0});
        ws_tokens += hi - lo;
      }
      tl = &tiles[t * kTileWords];
      tl[5] = (int32_t)cptr.size();
      for (int tok = 0; tok < tl[1]; ++tok) {
        cptr.push_back((int32_t)clist.size());
        for (int c = 0; c < (int)mine.size(); ++c) {
          const int32_t* cr = &contribs[(cbase + c) * kContribWords];
          if (tok >= cr[0] && tok < cr[1]) clist.push_back(c);
        }
      }
      cptr.push_back((int32_t)clist.size());
      const int rows = tl[1] * group();
      for (int r0 = 0; r0 < rows; r0 += kMergeRows) mblocks.insert(mblocks.end(), {t, r0});
    }
    for (auto& it : mine) {
      its.push_back(it);
      key_rows += it.cost * (int64_t)tl[1] * group();
    }
  }
  key_rows *= hkv;
  // longest items first (all KV heads of an item next to each other)
  std::stable_sort(its.begin(), its.end(), [](const ItemRec& a, const ItemRec& c) { return a.cost > c.cost; });
  for (auto& it : its)
    for (int h = 0; h < hkv; ++h) items.insert(items.end(), {it.tile, h, it.jb, it.je, it.c, 0, 0, 0});

  // ---- workspace ----
  const int64_t hq = desc.num_q_heads, d = desc.head_dim;
  // partial outputs [kvh][ws_token][grouped head][D] fp32, then (m, l) pairs
  ws_ml_offset = (ws_tokens * hq * d * 4 + 255) / 256 * 256;
  ws_bytes = num_split_tiles ? ws_ml_offset + ws_tokens * hq * 2 * 4 : 0;
  layout();
  built = true;
  return ok();
}

void Plan::layout() {
  int64_t w = 0;
  off_items = w; w = align16(w + (int64_t)items.size());
  off_tiles = w; w = align16(w + (int64_t)tiles.size());
  off_jobs = w; w = align16(w + (int64_t)jobs.size());
  off_toks = w; w = align16(w + (int64_t)toks.size());
  off_contribs = w; w = align16(w + (int64_t)contribs.size());
  off_runs = w; w = align16(w + (int64_t)runs.size());
  off_run_slots = w; w = align16(w + (int64_t)run_slots.size());
  off_new = w; w = align16(w + (int64_t)new_slots.size());
  off_cptr = w; w = align16(w + (int64_t)cptr.size());
  off_clist = w; w = align16(w + (int64_t)clist.size());
  off_mblocks = w; w = align16(w + (int64_t)mblocks.size());
  total_words = std::max<int64_t>(w, 16);
}

}  // namespace rdx
