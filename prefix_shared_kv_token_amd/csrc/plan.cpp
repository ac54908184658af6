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
#include <atomic>

#include "common.h"

namespace rdx {

namespace {

int64_t align16(int64_t w) { return (w + 15) & ~int64_t(15); }

struct Seg {
  int64_t start, end;  // key positions
  int rep;             // request whose page-table row is read for this segment
};

struct Req {
  int32_t row, kv_len, q_len, written, q_off, depth, shared_len;
  int64_t new_off;
  int32_t path_off, path_len;  // its root-to-node path in path_buf
  int32_t seg_off, seg_len;    // its shared segment ids (top-down) in seg_buf
};

struct TileReq {
  int r, lo, hi;  // request, its tile-local token range
  int32_t pmax;   // the position of its last token in the tile
};

struct Job {
  int32_t row, k0, k1, lo, hi, causal;
};

// Build scratch, reused across builds on a thread so a decode step does not
// allocate.
struct Scratch {
  std::vector<Req> rq;
  std::vector<const Node*> path_buf;
  std::vector<int> seg_buf, order, seen, tile_tr_begin, tile_job_begin;
  std::vector<Seg> segs;
  std::vector<TileReq> trs;
  std::vector<Job> tjobs, shared;
  std::vector<int32_t> row_set;  // open addressing: request index, -1 empty
};
thread_local Scratch g_scratch;
std::atomic<int64_t> g_epoch{0};

uint32_t hash_row(int32_t row) { return (uint32_t)row * 2654435761u; }

}  // namespace

int Plan::build(const RadixTree& tree, const rdx_batch& b, int64_t page_ld) {
  built = false;
  if (b.num_reqs < 0 || (b.num_reqs > 0 && (!b.node || !b.row || !b.kv_len || !b.q_len || !b.written)))
    return fail(RDX_EINVAL, "rdx_plan_build: bad batch pointers");
  if (page_ld <= 0 || page_ld > (int64_t)1 << 30) return fail(RDX_EINVAL, "rdx_plan_build: bad page-table stride");
  const int R = b.num_reqs;
  Scratch& sc = g_scratch;
  const int64_t ep = ++g_epoch;
  std::vector<Req>& rq = sc.rq;
  rq.resize(R);
  sc.path_buf.clear();
  // duplicate page-table rows: open-addressing set of request indices
  uint32_t cap = 16;
  while (cap < 2u * (uint32_t)R) cap <<= 1;
  sc.row_set.assign(cap, -1);
  int64_t total_new = 0;
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
    q.path_off = (int32_t)sc.path_buf.size();
    for (const Node* p = n; p != tree.root(); p = p->parent) {
      sc.path_buf.push_back(p);
      if (p->plan_epoch != ep) {
        p->plan_epoch = ep;
        p->plan_count = 0;
        p->plan_seg = -1;
      }
      p->plan_count++;
    }
    q.path_len = (int32_t)sc.path_buf.size() - q.path_off;
    std::reverse(sc.path_buf.begin() + q.path_off, sc.path_buf.end());
    q.depth = n == tree.root() ? 0 : (int32_t)n->end();
    const int64_t first_new = (int64_t)q.kv_len - q.q_len;
    if (q.row < 0 || q.q_len < 0 || q.q_len > q.kv_len || q.kv_len > page_ld || q.depth > first_new ||
        q.written < 0 || q.written > first_new || (q.written < first_new && q.depth < first_new))
      return fail(RDX_EINVAL,
                  "rdx_plan_build: request %d inconsistent (row %d kv_len %d q_len %d written %d cached %d)", r,
                  q.row, q.kv_len, q.q_len, q.written, q.depth);
    for (uint32_t h = hash_row(q.row) & (cap - 1);; h = (h + 1) & (cap - 1)) {
      const int32_t o = sc.row_set[h];
      if (o < 0) {
        sc.row_set[h] = r;
        break;
      }
      if (rq[o].row == q.row)
        return fail(RDX_EINVAL, "rdx_plan_build: requests %d and %d share page-table row %d", o, r, q.row);
    }
    max_page_row = std::max<int64_t>(max_page_row, q.row);
    total_new += q.q_len;
    if (total_new > ((int64_t)1 << 30)) return fail(RDX_EINVAL, "rdx_plan_build: too many new tokens");
  }
  if (total_new > 0 && !b.new_slots) return fail(RDX_EINVAL, "rdx_plan_build: new_slots missing");
  for (int64_t i = 0; i < total_new; ++i)
    if (b.new_slots[i] < 0 || b.new_slots[i] >= desc.num_slots)
      return fail(RDX_EINVAL, "rdx_plan_build: new slot %d out of range", b.new_slots[i]);

  // ---- sharing: nodes reached by >= 2 requests, grouped into segments ----
  std::vector<Seg>& segs = sc.segs;
  segs.clear();
  sc.seg_buf.clear();
  for (auto& q : rq) {
    const Node* const* path = sc.path_buf.data() + q.path_off;
    q.seg_off = (int32_t)sc.seg_buf.size();
    int i = 0;
    while (i < q.path_len && path[i]->plan_count >= 2) {
      int j = i;
      while (j + 1 < q.path_len && path[j + 1]->plan_count == path[i]->plan_count) ++j;
      int s = path[i]->plan_seg;
      if (s < 0) {
        s = (int)segs.size();
        segs.push_back({path[i]->start, path[j]->end(), -1});
        path[i]->plan_seg = s;
      }
      sc.seg_buf.push_back(s);
      i = j + 1;
    }
    q.seg_len = (int32_t)sc.seg_buf.size() - q.seg_off;
    q.shared_len = q.seg_len == 0 ? 0 : (int32_t)segs[sc.seg_buf[q.seg_off + q.seg_len - 1]].end;
  }
  num_shared_segments = (int64_t)segs.size();

  // ---- depth-first order: lexicographic on segment lists (stable) ----
  std::vector<int>& order = sc.order;
  order.resize(R);
  for (int r = 0; r < R; ++r) order[r] = r;
  const int* sb = sc.seg_buf.data();
  auto seg_less = [&](int a, int c) {
    const Req& x = rq[a];
    const Req& y = rq[c];
    return std::lexicographical_compare(sb + x.seg_off, sb + x.seg_off + x.seg_len, sb + y.seg_off,
                                        sb + y.seg_off + y.seg_len);
  };
  // batches usually arrive grouped already (admission order)
  if (!std::is_sorted(order.begin(), order.end(), seg_less)) std::stable_sort(order.begin(), order.end(), seg_less);
  for (int r : order)
    for (int k = 0; k < rq[r].seg_len; ++k) {
      Seg& sg = segs[sb[rq[r].seg_off + k]];
      if (sg.rep < 0) sg.rep = r;
    }

  // ---- page-table writes: [written, kv_len) of each row ----
  runs.clear();
  run_slots.clear();
  for (int r = 0; r < R; ++r) {
    const Req& q = rq[r];
    if (q.written >= q.kv_len) continue;
    int64_t src = (int64_t)run_slots.size();
    const Node* const* path = sc.path_buf.data() + q.path_off;
    for (int k = 0; k < q.path_len; ++k) {
      const Node* n = path[k];
      const int64_t p0 = std::max<int64_t>(n->start, q.written);
      if (p0 < n->end())
        run_slots.insert(run_slots.end(), n->slots.begin() + (p0 - n->start), n->slots.begin() + (n->end() - n->start));
    }
    const int64_t i0 = std::max<int64_t>(0, (int64_t)q.written - (q.kv_len - q.q_len));
    if (i0 < q.q_len)
      run_slots.insert(run_slots.end(), b.new_slots + q.new_off + i0, b.new_slots + q.new_off + q.q_len);
    int64_t count = (int64_t)run_slots.size() - src;
    if (count != q.kv_len - q.written) return fail(RDX_EINVAL, "rdx_plan_build: request %d: page-table gap", r);
    runs.insert(runs.end(), {q.row, q.written, (int32_t)count, (int32_t)src});
  }
  new_slots.assign(b.new_slots, b.new_slots + total_new);

  // ---- tiles ----
  const int tt = tile_tokens();
  toks.clear();
  tiles.clear();
  sc.trs.clear();
  sc.tile_tr_begin.clear();
  int64_t cur_key = INT64_MIN, cur_key2 = INT64_MIN;
  // decode tiles hold one top-level sharing group; inside it, a run of
  // requests that also share their next segment (a branch of the tree) starts
  // a fresh tile when it would not fit in the current one but fits in a
  // tile of its own, so that no branch is streamed by two tiles
  auto key2_of = [&](const Req& q) -> int64_t { return q.seg_len < 2 ? -1 : sb[q.seg_off + 1]; };
  for (int oi = 0; oi < R; ++oi) {
    const int r = order[oi];
    const Req& q = rq[r];
    if (q.q_len == 0) continue;
    int64_t key, key2 = -1;
    if (kind == RDX_PLAN_EXTEND) {
      key = q.seg_len == 0 ? -1 - (int64_t)r : sb[q.seg_off + q.seg_len - 1];
    } else {
      key = q.seg_len == 0 ? -1 : sb[q.seg_off];
      key2 = key2_of(q);
      const int ntile = (int)sc.tile_tr_begin.size();
      if (key2 >= 0 && ntile > 0 && key == cur_key && key2 != cur_key2) {
        int64_t run = 0;
        for (int oj = oi; oj < R; ++oj) {
          const Req& x = rq[order[oj]];
          if (x.seg_len < 1 || sb[x.seg_off] != key || key2_of(x) != key2) break;
          run += x.q_len;
        }
        const int used = tiles[(ntile - 1) * kTileWords + 1];
        if (used > 0 && used + run > tt && run <= tt) cur_key = INT64_MIN;  // forces a fresh tile
      }
      cur_key2 = key2;
    }
    // the request's tokens in runs that fill the current tile
    for (int t = 0; t < q.q_len;) {
      int ntile = (int)sc.tile_tr_begin.size();
      bool fresh = ntile == 0 || key != cur_key || tiles[(ntile - 1) * kTileWords + 1] >= tt;
      if (fresh) {
        tiles.insert(tiles.end(), {(int32_t)(toks.size() / kTokWords), 0, 0, 0, -1, 0, 0, 0});
        sc.tile_tr_begin.push_back((int)sc.trs.size());
        cur_key = key;
        ntile++;
      }
      int32_t* tl = &tiles[(ntile - 1) * kTileWords];
      const int local = tl[1];
      const int n = std::min(q.q_len - t, tt - local);
      if ((int)sc.trs.size() == sc.tile_tr_begin.back() || sc.trs.back().r != r) sc.trs.push_back({r, local, local, 0});
      sc.trs.back().hi = local + n;
      sc.trs.back().pmax = q.kv_len - q.q_len + t + n - 1;
      tl[1] += n;
      const size_t at = toks.size();
      toks.resize(at + (size_t)n * kTokWords);
      int32_t* out = toks.data() + at;
      const int32_t qi = q.q_off + t, pos = q.kv_len - q.q_len + t;
      for (int i = 0; i < n; ++i) {
        out[2 * i] = qi + i;
        out[2 * i + 1] = pos + i;
      }
      t += n;
    }
  }
  const int ntiles = (int)sc.tile_tr_begin.size();
  sc.tile_tr_begin.push_back((int)sc.trs.size());

  // ---- jobs per tile (before splitting): its shared segments, then each
  // request's own causal range ----
  sc.tjobs.clear();
  sc.tile_job_begin.clear();
  int64_t total_cost = 0;
  for (int t = 0; t < ntiles; ++t) {
    sc.tile_job_begin.push_back((int)sc.tjobs.size());
    sc.seen.clear();
    sc.shared.clear();
    for (int k = sc.tile_tr_begin[t]; k < sc.tile_tr_begin[t + 1]; ++k) {
      const TileReq& tr = sc.trs[k];
      const Req& q = rq[tr.r];
      for (int m = 0; m < q.seg_len; ++m) {
        const int s = sb[q.seg_off + m];
        auto it = std::find(sc.seen.begin(), sc.seen.end(), s);
        if (it == sc.seen.end()) {
          sc.seen.push_back(s);
          sc.shared.push_back({rq[segs[s].rep].row, (int32_t)segs[s].start, (int32_t)segs[s].end, tr.lo, tr.hi, 0});
        } else {
          Job& j = sc.shared[it - sc.seen.begin()];
          j.lo = std::min(j.lo, tr.lo);
          j.hi = std::max(j.hi, tr.hi);
        }
      }
    }
    sc.tjobs.insert(sc.tjobs.end(), sc.shared.begin(), sc.shared.end());
    for (int k = sc.tile_tr_begin[t]; k < sc.tile_tr_begin[t + 1]; ++k) {
      const TileReq& tr = sc.trs[k];
      const Req& q = rq[tr.r];
      // causal: no token of this tile sees keys past its last position, so
      // the job ends there (a causal prefill tile reads only the blocks up
      // to its diagonal)
      if (q.kv_len > q.shared_len)
        sc.tjobs.push_back({q.row, q.shared_len, std::min(q.kv_len, tr.pmax + 1), tr.lo, tr.hi, 1});
    }
  }
  sc.tile_job_begin.push_back((int)sc.tjobs.size());
  // cost unit: 64-key blocks (a block costs about the same whether or not
  // all its keys exist: the same MFMA work in extend, about one memory round
  // trip in decode)
  for (const Job& j : sc.tjobs) total_cost += (j.k1 - j.k0 + kKeyBlock - 1) / kKeyBlock;

  // ---- split into items ----
  const int hkv = desc.num_kv_heads;
  // default launch size the split aims for (about one round of workgroups):
  // extend splits only when fewer work items than that exist -- 256 for the
  // 256-row kernel (one workgroup per CU), 512 for the 128-row one (two);
  // decode aims for whole workgroups per CU on every XCD (a launch whose
  // items leave some CUs of an XCD one workgroup more than others runs at
  // the pace of those): two per CU when an item would be short (the second
  // workgroup's stream covers the first's start-up), one per CU when each
  // item gets at least 32 blocks that way (the start-up is amortised, and
  // half the items means half the partials to write and merge).  Measured on
  // MI355X: 1,000-key prefix + 64 short requests best at 512 (items of 9
  // blocks), 16,000-key prefixes at 256 (items of 42 blocks)
  int64_t target = target_items > 0 ? target_items : (kind == RDX_PLAN_EXTEND && tile_rows == 256 ? 256 : 512);
  if (target_items <= 0 && kind == RDX_PLAN_DECODE) {
    const int64_t per_kvh1 = std::max<int64_t>(1, 256 / hkv);
    if ((total_cost + per_kvh1 - 1) / per_kvh1 >= 32) target = 256;
  }
  // blocks per tile
  static thread_local std::vector<int64_t> tcost;
  tcost.assign(ntiles, 0);
  for (int t = 0; t < ntiles; ++t)
    for (int jx = sc.tile_job_begin[t]; jx < sc.tile_job_begin[t + 1]; ++jx)
      tcost[t] += (sc.tjobs[jx].k1 - sc.tjobs[jx].k0 + kKeyBlock - 1) / kKeyBlock;
  // items per tile (each tile's blocks are cut into that many runs of
  // nearly equal length)
  static thread_local std::vector<int64_t> npieces;
  npieces.assign(ntiles, 1);
  const int64_t per_kvh = std::max<int64_t>(1, target / hkv);
  if ((int64_t)ntiles * hkv < target && total_cost > 0) {
    // fewer tiles than the target: hand out the target's items one at a
    // time to the tile whose pieces are currently the longest (the launch
    // takes as long as its longest item), never more pieces than blocks.
    // The count is exact, so items per XCD stay a whole number per CU
    // (an item count a little over a multiple of the CU count would start a
    // second round of workgroups for a few of them)
    static thread_local std::vector<std::pair<int64_t, int>> heap;
    heap.clear();
    auto piece = [&](int t) { return (tcost[t] + npieces[t] - 1) / npieces[t]; };
    for (int t = 0; t < ntiles; ++t) heap.push_back({piece(t), t});
    std::make_heap(heap.begin(), heap.end());
    for (int64_t given = ntiles; given < per_kvh && !heap.empty();) {
      std::pop_heap(heap.begin(), heap.end());
      const int t = heap.back().second;
      heap.pop_back();
      if (npieces[t] >= tcost[t]) continue;  // one block per piece: no further cut
      ++npieces[t];
      ++given;
      heap.push_back({piece(t), t});
      std::push_heap(heap.begin(), heap.end());
    }
  } else if (ntiles > per_kvh && ntiles % per_kvh != 0 && per_kvh / (ntiles % per_kvh) >= 4 &&
             *std::max_element(tcost.begin(), tcost.end()) <= 2 * *std::min_element(tcost.begin(), tcost.end())) {
    // more tiles than one round of workgroups, of similar cost (within 2x),
    // and a short last round of e tiles per KV head: that round would leave
    // most CUs idle for a whole tile's time (tiles of varied cost, as in a
    // causal prefill, even out by longest-first dispatch instead).  The last e tiles (dispatched last) are cut into
    // per_kvh / e pieces each, so the last round is full with pieces of a
    // quarter of a tile or less.  Measured on MI355X (extend, 256-row
    // tiles): 10 tiles per head on 8 slots, last 2 in quarters, 116 -> 98 us
    // with the merge; 48 on 32, last 16 in halves, no gain (134 -> 137 us:
    // the merge and the partial writes eat the half round)
    const int64_t e = ntiles % per_kvh;
    for (int t = ntiles - (int)e; t < ntiles; ++t) npieces[t] = std::min(per_kvh / e, std::max<int64_t>(1, tcost[t]));
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
  struct ItemRec { int32_t tile, jb, je, c; int64_t cost, keys; };
  static thread_local std::vector<ItemRec> its, mine;
  its.clear();
  for (int t = 0; t < ntiles; ++t) {
    int32_t* tl = &tiles[t * kTileWords];
    mine.clear();
    // item i of the tile ends at block floor((i + 1) cost / n)
    const int64_t np = npieces[t], ct = tcost[t];
    int64_t used = 0;
    auto item_end = [&](int64_t i) { return (i + 1) * ct / np; };
    for (int jx = sc.tile_job_begin[t]; jx < sc.tile_job_begin[t + 1]; ++jx) {
      const Job& j = sc.tjobs[jx];
      for (int64_t a = j.k0; a < j.k1;) {
        int64_t room = mine.empty() ? 0 : item_end((int64_t)mine.size() - 1) - used;
        if (room <= 0) {
          mine.push_back({t, (int32_t)(jobs.size() / kJobWords), (int32_t)(jobs.size() / kJobWords),
                          (int32_t)mine.size(), 0, 0});
          room = item_end((int64_t)mine.size() - 1) - used;
        }
        // room is in blocks: the piece takes whole blocks of the job
        const int64_t e = room >= ((int64_t)j.k1 - a + kKeyBlock - 1) / kKeyBlock ? (int64_t)j.k1 : a + room * kKeyBlock;
        const int64_t nb = (e - a + kKeyBlock - 1) / kKeyBlock;
        jobs.insert(jobs.end(), {j.row, (int32_t)a, (int32_t)e, j.lo, j.hi, j.causal, 0, 0});
        mine.back().je++;
        mine.back().cost += nb;
        mine.back().keys += e - a;
        used += nb;
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
          if (tok >= cr[0] && tok < cr[1]) clist.push_back(cr[2] + tok - cr[0]);  // its workspace token
        }
      }
      cptr.push_back((int32_t)clist.size());
      const int rows = tl[1] * group();
      for (int r0 = 0; r0 < rows; r0 += kMergeRows) {
        const int t0 = r0 / group();
        int32_t rec[kMBlockWords] = {r0, tl[1], tl[0], t0};
        for (int i = 0; i <= kMergeRows; ++i) rec[4 + i] = cptr[tl[5] + std::min(t0 + i, (int)tl[1])];
        mblocks.insert(mblocks.end(), rec, rec + kMBlockWords);
      }
    }
    for (auto& it : mine) {
      its.push_back(it);
      key_rows += it.keys * (int64_t)tl[1] * group();
    }
  }
  key_rows *= hkv;
  // Dispatch order (all KV heads of an item next to each other).  Items are
  // grouped by the key stream their tile starts with -- the page-table row
  // of its first job: a shared prefix, or the request's own causal range --
  // streams ordered by their longest item (then first appearance), and
  // within a stream the longest items first.  Workgroup i*Hkv + h runs on
  // XCD (i*Hkv + h) mod 8, so the items one XCD runs at a time are
  // consecutive records: grouped by stream they read the same keys at
  // about the same time and share that XCD's L2.  Ordered by length alone,
  // a causal prefill interleaves every sequence's longest tiles, and each
  // of an XCD's workgroups streams a different sequence.
  {
    static thread_local std::vector<int64_t> key_of_tile, smax, sfirst;
    key_of_tile.assign(ntiles, 0);
    smax.clear();
    sfirst.clear();
    // stream index per tile: consecutive tiles with the same first-job row
    // share one (a stream's tiles are consecutive: requests are ordered by
    // their segments, a request's tiles follow each other)
    int32_t prev_row = INT32_MIN;
    for (int t = 0; t < ntiles; ++t) {
      const int32_t row = sc.tile_job_begin[t] == sc.tile_job_begin[t + 1] ? INT32_MIN + 1 + t
                                                                          : sc.tjobs[sc.tile_job_begin[t]].row;
      if (t == 0 || row != prev_row) {
        smax.push_back(0);
        sfirst.push_back(t);
      }
      prev_row = row;
      key_of_tile[t] = (int64_t)smax.size() - 1;
    }
    for (auto& it : its) smax[key_of_tile[it.tile]] = std::max<int64_t>(smax[key_of_tile[it.tile]], it.cost);
    std::stable_sort(its.begin(), its.end(), [&](const ItemRec& a, const ItemRec& c) {
      const int64_t sa = key_of_tile[a.tile], sb = key_of_tile[c.tile];
      if (sa != sb) return smax[sa] != smax[sb] ? smax[sa] > smax[sb] : sfirst[sa] < sfirst[sb];
      return a.cost > c.cost;
    });
  }
  // one record per chunk; the launch runs record i for KV heads 0..Hkv-1 as
  // workgroups i*Hkv .. i*Hkv+Hkv-1
  for (auto& it : its) {
    const int32_t* tl = &tiles[(int64_t)it.tile * kTileWords];
    int32_t nb = 0;
    for (int32_t jx = it.jb; jx < it.je; ++jx) nb += (jobs[jx * kJobWords + 2] - jobs[jx * kJobWords + 1] + 63) / 64;
    int32_t lo = 0, hi = tl[1], base = 0;
    if (tl[4] >= 0) {
      const int32_t* cr = &contribs[(int64_t)(tl[3] + it.c) * kContribWords];
      lo = cr[0];
      hi = cr[1];
      base = cr[2];
    }
    const int32_t* j0 = &jobs[(int64_t)it.jb * kJobWords];
    // the tile's first caller Q row when its tokens' rows are consecutive
    // (the kernels then address Q without the token records), else -1
    int32_t q0 = toks[(int64_t)tl[0] * kTokWords];
    for (int32_t k = 1; k < tl[1] && q0 >= 0; ++k)
      if (toks[(int64_t)(tl[0] + k) * kTokWords] != q0 + k) q0 = -1;
    items.insert(items.end(), {it.tile, it.jb, it.je, it.c, nb, tl[0], tl[1], tl[4], lo, hi, base, j0[0], j0[1],
                               j0[2], j0[3], j0[4], j0[5], q0, 0, 0});
  }

  // ---- workspace ----
  const int64_t hq = desc.num_q_heads, d = desc.head_dim;
  // partial outputs [kvh][ws_token][grouped head][D] fp32, then (m, l) pairs
  ws_ml_offset = (ws_tokens * hq * d * 4 + 255) / 256 * 256;
  ws_bytes = num_split_tiles ? ws_ml_offset + ws_tokens * hq * 2 * 4 : 0;
  layout();
  built = true;
  return ok();
}

void Plan::fill_info(rdx_plan_info* out) const {
  out->device_bytes = total_words * 4;
  out->workspace_bytes = ws_bytes;
  out->new_slots_offset = off_new * 4;
  out->num_new = (int64_t)new_slots.size();
  out->num_items = (int64_t)items.size() / kItemWords * desc.num_kv_heads;
  out->num_tiles = (int64_t)tiles.size() / kTileWords;
  out->num_jobs = (int64_t)jobs.size() / kJobWords;
  out->num_split_tiles = num_split_tiles;
  out->num_shared_segments = num_shared_segments;
  out->key_rows = key_rows;
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
