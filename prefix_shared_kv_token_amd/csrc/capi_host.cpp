// C ABI: host-side entry points (tree, planner).  The device entry points
// live in device.hip.
#include <cmath>
#include <cstring>
#include <new>
#include <string>

#include "common.h"
#include "plan.h"
#include "radix_tree.h"

namespace rdx {
std::string& last_error() {
  thread_local std::string msg;
  return msg;
}
}  // namespace rdx

using rdx::fail;

extern "C" {

const char* rdx_last_error(void) { return rdx::last_error().c_str(); }
const char* rdx_version(void) { return "rdx 0.1 gfx950"; }

int rdx_tree_create(int64_t num_slots, int32_t match_unit, rdx_tree** out) {
  if (!out || num_slots <= 0 || num_slots >= ((int64_t)1 << 31) || match_unit < 1)
    return fail(RDX_EINVAL, "rdx_tree_create: need 0 < num_slots < 2^31 and match_unit >= 1");
  try {
    *out = new rdx_tree(num_slots, match_unit);
  } catch (const std::bad_alloc&) {
    return fail(RDX_EINVAL, "rdx_tree_create: out of host memory");
  }
  return rdx::ok();
}

void rdx_tree_destroy(rdx_tree* tree) { delete tree; }

int rdx_match_prefix(rdx_tree* t, const int32_t* tokens, int64_t n, int32_t* out_slots, int64_t* out_len,
                     int64_t* out_node) {
  if (!t) return fail(RDX_EINVAL, "rdx_match_prefix: null tree");
  return t->impl.match_prefix(tokens, n, out_slots, out_len, out_node);
}

int rdx_lock(rdx_tree* t, int64_t node) {
  if (!t) return fail(RDX_EINVAL, "rdx_lock: null tree");
  return t->impl.lock(node);
}

int rdx_unlock(rdx_tree* t, int64_t node) {
  if (!t) return fail(RDX_EINVAL, "rdx_unlock: null tree");
  return t->impl.unlock(node);
}

int rdx_alloc(rdx_tree* t, int64_t n, int32_t* out_slots) {
  if (!t) return fail(RDX_EINVAL, "rdx_alloc: null tree");
  return t->impl.alloc(n, out_slots);
}

int rdx_free(rdx_tree* t, const int32_t* slots, int64_t n) {
  if (!t) return fail(RDX_EINVAL, "rdx_free: null tree");
  return t->impl.free_slots(slots, n);
}

int rdx_insert(rdx_tree* t, const int32_t* tokens, const int32_t* slots, int64_t n, int64_t* out_present,
               int64_t* out_node) {
  if (!t) return fail(RDX_EINVAL, "rdx_insert: null tree");
  return t->impl.insert(tokens, slots, n, out_present, out_node);
}

int rdx_evict(rdx_tree* t, int64_t n_tokens, int64_t* out_freed) {
  if (!t) return fail(RDX_EINVAL, "rdx_evict: null tree");
  return t->impl.evict(n_tokens, out_freed);
}

int rdx_admit(rdx_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* offsets, const int32_t* rows,
              int32_t* host_page_table, int64_t num_rows, int64_t ld, int64_t* out_matched, int64_t* out_node,
              int32_t* out_new_slots, int32_t* out_admitted) {
  if (!t || !out_admitted || num_reqs < 0 || num_rows <= 0 || ld <= 0)
    return fail(RDX_EINVAL, "rdx_admit: bad arguments");
  *out_admitted = 0;
  if (num_reqs == 0) return rdx::ok();
  if (!tokens || !offsets || !rows || !host_page_table || !out_matched || !out_node || !out_new_slots)
    return fail(RDX_EINVAL, "rdx_admit: null array");
  rdx::RadixTree& tr = t->impl;
  int64_t nn = 0;  // new slots written so far
  for (int32_t i = 0; i < num_reqs; ++i) {
    const int64_t n = offsets[i + 1] - offsets[i];
    const int32_t r = rows[i];
    if (n < 0 || n > ld || r < 0 || r >= num_rows)
      return fail(RDX_EINVAL, "rdx_admit: request %d: length %lld, row %d (ld %lld, %lld rows)", i, (long long)n, r,
                  (long long)ld, (long long)num_rows);
    int32_t* row = host_page_table + (int64_t)r * ld;
    int64_t m = 0, node = 0;
    int rc = tr.match_prefix(tokens + offsets[i], n, row, &m, &node);
    if (rc) return rc;
    rc = tr.lock(node);
    if (rc) return rc;
    rc = tr.alloc(n - m, row + m);
    if (rc) {
      const std::string msg = rdx::last_error();
      tr.unlock(node);
      rdx::last_error() = msg;
      return rc;
    }
    std::memcpy(out_new_slots + nn, row + m, (size_t)(n - m) * sizeof(int32_t));
    nn += n - m;
    out_matched[i] = m;
    out_node[i] = node;
    *out_admitted = i + 1;
  }
  return rdx::ok();
}

int rdx_finish(rdx_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* offsets, const int32_t* rows,
               const int32_t* host_page_table, int64_t num_rows, int64_t ld, const int64_t* matched,
               const int64_t* node, int32_t* out_done) {
  if (!t || !out_done || num_reqs < 0 || num_rows <= 0 || ld <= 0) return fail(RDX_EINVAL, "rdx_finish: bad arguments");
  *out_done = 0;
  if (num_reqs == 0) return rdx::ok();
  if (!tokens || !offsets || !rows || !host_page_table || !matched || !node)
    return fail(RDX_EINVAL, "rdx_finish: null array");
  rdx::RadixTree& tr = t->impl;
  for (int32_t i = 0; i < num_reqs; ++i) {
    const int64_t n = offsets[i + 1] - offsets[i];
    const int32_t r = rows[i];
    if (n < 0 || n > ld || r < 0 || r >= num_rows || matched[i] < 0 || matched[i] > n)
      return fail(RDX_EINVAL, "rdx_finish: request %d: length %lld, row %d, matched %lld", i, (long long)n, r,
                  (long long)matched[i]);
    const int32_t* row = host_page_table + (int64_t)r * ld;
    int64_t present = 0, nd = 0;
    int rc = tr.insert(tokens + offsets[i], row, n, &present, &nd);
    if (rc) return rc;
    if (present > matched[i]) {
      rc = tr.free_slots(row + matched[i], present - matched[i]);
      if (rc) return rc;
    }
    rc = tr.unlock(node[i]);
    if (rc) return rc;
    *out_done = i + 1;
  }
  return rdx::ok();
}

int rdx_tree_stats(const rdx_tree* t, rdx_stats* out) {
  if (!t || !out) return fail(RDX_EINVAL, "rdx_tree_stats: null argument");
  const auto& x = t->impl;
  out->num_slots = x.num_slots();
  out->free = x.num_free();
  out->cached = x.count_state(rdx::RadixTree::kTree);
  out->evictable = x.evictable_tokens();
  out->private_ = x.count_state(rdx::RadixTree::kPrivate);
  out->nodes = x.num_nodes();
  out->evictions = x.evictions();
  out->clock = x.clock();
  return rdx::ok();
}

int rdx_tree_set_policy(rdx_tree* t, int32_t policy) {
  if (!t) return fail(RDX_EINVAL, "rdx_tree_set_policy: null tree");
  return t->impl.set_policy(policy);
}

int rdx_tree_set_priority(rdx_tree* t, int32_t priority) {
  if (!t) return fail(RDX_EINVAL, "rdx_tree_set_priority: null tree");
  t->impl.set_priority(priority);
  return rdx::ok();
}

int rdx_node_get(const rdx_tree* t, int64_t node, rdx_node_info* out, int32_t* out_slots) {
  if (!t || !out) return fail(RDX_EINVAL, "rdx_node_get: null argument");
  const rdx::Node* n = t->impl.find(node);
  if (!n) return fail(RDX_ESTATE, "rdx_node_get: unknown node %lld", (long long)node);
  out->id = n->id;
  out->parent = (n->parent == nullptr || n->parent == t->impl.root()) ? 0 : n->parent->id;
  out->start = n->start;
  out->length = (int64_t)n->key.size();
  out->ref = n->ref;
  out->last_access = n->last_access;
  out->num_children = (int64_t)n->children.size();
  out->hits = n->hits;
  out->priority = n->prio;
  if (out_slots)
    for (size_t i = 0; i < n->slots.size(); ++i) out_slots[i] = n->slots[i];
  return rdx::ok();
}

int rdx_plan_create(const rdx_attn_desc* desc, int32_t kind, int32_t target_items, rdx_plan** out) {
  if (!out || !desc) return fail(RDX_EINVAL, "rdx_plan_create: null argument");
  if (kind != RDX_PLAN_EXTEND && kind != RDX_PLAN_DECODE) return fail(RDX_EINVAL, "rdx_plan_create: bad kind %d", kind);
  if (target_items < 0) return fail(RDX_EINVAL, "rdx_plan_create: negative target_items");
  int rc = rdx::check_desc(desc);
  if (rc) return rc;
  auto* p = new (std::nothrow) rdx::Plan();
  if (!p) return fail(RDX_EINVAL, "rdx_plan_create: out of host memory");
  p->desc = *desc;
  p->kind = kind;
  p->target_items = target_items;
  if (kind == RDX_PLAN_DECODE) p->n_stages = rdx::Plan::kMaxStages;
  if (kind == RDX_PLAN_EXTEND && desc->dtype == RDX_BF16 && desc->head_dim == 128) p->tile_rows = 2 * rdx::kTileRows;
  // bf16 decode: 64-row tiles for the decode kernel (a group's new tokens x
  // the GQA group fit one tile whenever the group has at most 64 heads)
  if (kind == RDX_PLAN_DECODE && desc->dtype == RDX_BF16 && desc->num_q_heads / desc->num_kv_heads <= 64)
    p->tile_rows = rdx::kDecodeTileRows;
  *out = reinterpret_cast<rdx_plan*>(p);
  return rdx::ok();
}

int rdx_plan_build(rdx_plan* plan, const rdx_tree* tree, const rdx_batch* batch, int64_t ld) {
  if (!plan || !tree || !batch) return fail(RDX_EINVAL, "rdx_plan_build: null argument");
  auto* p = reinterpret_cast<rdx::Plan*>(plan);
  p->ld = ld;
  return p->build(tree->impl, *batch, ld);
}

int rdx_plan_get_info(const rdx_plan* plan, rdx_plan_info* out) {
  if (!plan || !out) return fail(RDX_EINVAL, "rdx_plan_get_info: null argument");
  auto* p = reinterpret_cast<const rdx::Plan*>(plan);
  if (!p->built) return fail(RDX_ESTATE, "rdx_plan_get_info: plan not built");
  p->fill_info(out);
  return rdx::ok();
}

int rdx_plan_get_view(const rdx_plan* plan, rdx_plan_view* out) {
  if (!plan || !out) return fail(RDX_EINVAL, "rdx_plan_get_view: null argument");
  auto* p = reinterpret_cast<const rdx::Plan*>(plan);
  if (!p->built) return fail(RDX_ESTATE, "rdx_plan_get_view: plan not built");
  out->items = p->items.data();
  out->num_items = (int64_t)p->items.size() / rdx::kItemWords;
  out->tiles = p->tiles.data();
  out->num_tiles = (int64_t)p->tiles.size() / rdx::kTileWords;
  out->jobs = p->jobs.data();
  out->num_jobs = (int64_t)p->jobs.size() / rdx::kJobWords;
  out->tokens = p->toks.data();
  out->num_tokens = (int64_t)p->toks.size() / rdx::kTokWords;
  out->contribs = p->contribs.data();
  out->num_contribs = (int64_t)p->contribs.size() / rdx::kContribWords;
  out->tile_rows = p->tile_rows;
  out->group = p->group();
  return rdx::ok();
}

}  // extern "C"

namespace rdx {
int check_desc(const rdx_attn_desc* d) {
  if (!d) return fail(RDX_EINVAL, "null attention descriptor");
  if (d->dtype != RDX_F32 && d->dtype != RDX_BF16) return fail(RDX_EUNSUPPORTED, "dtype %d not supported", d->dtype);
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads)
    return fail(RDX_EINVAL, "heads: need Hkv > 0 dividing Hq (got %d/%d)", d->num_q_heads, d->num_kv_heads);
  int g = d->num_q_heads / d->num_kv_heads;
  if (g > kTileRows || kTileRows % g) return fail(RDX_EUNSUPPORTED, "Hq/Hkv = %d must divide %d", g, kTileRows);
  if (d->head_dim != 64 && d->head_dim != 128) return fail(RDX_EUNSUPPORTED, "head_dim %d (64 or 128)", d->head_dim);
  if (d->num_slots <= 0 || d->num_slots >= ((int64_t)1 << 31)) return fail(RDX_EINVAL, "num_slots out of range");
  if (!(d->sm_scale >= 0.f) || std::isinf(d->sm_scale)) return fail(RDX_EINVAL, "sm_scale must be finite and >= 0");
  if (d->kv_row_pitch < 0 || (d->kv_row_pitch > 0 && (d->kv_row_pitch < (int64_t)d->num_kv_heads * d->head_dim ||
                                                       (d->kv_row_pitch * kv_elem_bytes(d)) % 16)))
    return fail(RDX_EINVAL, "kv_row_pitch %d: 0, or >= Hkv*head_dim with 16-byte rows", d->kv_row_pitch);
  return ok();
}
}  // namespace rdx

int rdx_kv_row_pitch_recommended(const rdx_attn_desc* desc, int32_t* out) {
  if (!desc || !out) return fail(RDX_EINVAL, "rdx_kv_row_pitch_recommended: null argument");
  rdx_attn_desc d = *desc;
  d.kv_row_pitch = 0;
  int rc = rdx::check_desc(&d);
  if (rc) return rc;
  const int64_t es = rdx::kv_elem_bytes(&d), dense = (int64_t)d.num_kv_heads * d.head_dim;
  *out = (int32_t)((dense * es) % 1024 == 0 ? dense + 256 / es : dense);
  return rdx::ok();
}
