// Radix tree + slot allocator (see radix_tree.h for the passages followed).
//
// Readings of points the pages leave open (identical in the oracle):
//  * a match that ends inside an edge splits the edge there, so the node a
//    request locks covers exactly its matched tokens;
//  * the LRU clock ticks once per match/insert call and stamps every node on
//    the walked path; a split gives the upper part a new id (the next one),
//    the lower part's stamp and the same reference count, and the lower part
//    keeps its id and stamp;
//  * eviction takes whole unreferenced leaves, smallest (last access, id)
//    first, and repeats as parents become leaves;
//  * the other eviction orders (LFU, SLRU, priority; the pages name them
//    beside LRU): every stamp also counts one access and raises the node's
//    priority to the call's; a new node starts with one access and the
//    call's priority; a split's upper part copies both.  The victim is the
//    smallest (major, last access, id), major = accesses (LFU), protected =
//    accesses >= 2 (SLRU: probation goes first), priority (priority), 0 (LRU);
//  * allocation hands out the smallest free slot ids in ascending order and
//    evicts only the shortfall; it fails without side effects when free +
//    evictable slots cannot cover the request.
#include "radix_tree.h"

#include <algorithm>
#include <tuple>

#include "common.h"

namespace rdx {

RadixTree::RadixTree(int64_t num_slots, int32_t match_unit)
    : num_slots_(num_slots), unit_(match_unit), state_(num_slots, kFree),
      free_bits_((num_slots + 63) / 64, ~uint64_t(0)), n_free_(num_slots) {
  if (num_slots % 64) free_bits_.back() = (uint64_t(1) << (num_slots % 64)) - 1;
}

RadixTree::~RadixTree() = default;

const Node* RadixTree::find(int64_t id) const {
  if (id == 0) return &root_;
  auto it = nodes_.find(id);
  return it == nodes_.end() ? nullptr : it->second.get();
}

int64_t RadixTree::count_state(uint8_t s) const {
  return (int64_t)std::count(state_.begin(), state_.end(), s);
}

// Tokens of nodes with no referenced node at or below them: exactly those
// that repeated leaf eviction can reach.
int64_t RadixTree::evictable_tokens() const {
  std::unordered_map<const Node*, bool> pinned;
  for (auto& kv : nodes_) {
    if (kv.second->ref <= 0) continue;
    for (const Node* p = kv.second.get(); p != &root_ && !pinned.count(p); p = p->parent) pinned[p] = true;
  }
  int64_t t = 0;
  for (auto& kv : nodes_)
    if (!pinned.count(kv.second.get())) t += (int64_t)kv.second->key.size();
  return t;
}

int64_t RadixTree::walk(const int32_t* t, int64_t n, std::vector<WalkStep>* steps) {
  steps->clear();
  Node* cur = &root_;
  int64_t m = 0;
  while (m < n) {
    auto it = cur->children.find(t[m]);
    if (it == cur->children.end()) break;
    Node* c = it->second;
    const int64_t len = (int64_t)c->key.size();
    const int64_t l = common_prefix(c->key.data(), t + m, std::min(len, n - m));
    steps->push_back({c, l});
    m += l;
    if (l < len) break;
    cur = c;
  }
  return m;
}

int64_t RadixTree::peek_match(const int32_t* t, int64_t n) const {
  const Node* cur = &root_;
  int64_t m = 0;
  while (m < n) {
    auto it = cur->children.find(t[m]);
    if (it == cur->children.end()) break;
    const Node* c = it->second;
    const int64_t len = (int64_t)c->key.size();
    const int64_t l = common_prefix(c->key.data(), t + m, std::min(len, n - m));
    m += l;
    if (l < len) break;
    cur = c;
  }
  return (m / unit_) * unit_;
}

Node* RadixTree::split(Node* x, int64_t c) {
  auto y = std::make_unique<Node>();
  y->id = next_id_++;
  y->parent = x->parent;
  y->start = x->start;
  y->key.assign(x->key.begin(), x->key.begin() + c);
  y->slots.assign(x->slots.begin(), x->slots.begin() + c);
  y->last_access = x->last_access;
  y->ref = x->ref;
  y->hits = x->hits;
  y->prio = x->prio;
  x->key.erase(x->key.begin(), x->key.begin() + c);
  x->slots.erase(x->slots.begin(), x->slots.begin() + c);
  x->start += c;
  x->parent = y.get();
  y->children[x->key[0]] = x;
  y->parent->children[y->key[0]] = y.get();
  Node* out = y.get();
  nodes_[out->id] = std::move(y);
  return out;
}

Node* RadixTree::node_ending_at(const std::vector<WalkStep>& steps, int64_t d) {
  for (const WalkStep& s : steps) {
    Node* x = s.node;
    if (d <= x->end()) return d == x->end() ? x : split(x, d - x->start);
  }
  return nullptr;  // unreachable when d <= matched length
}

void RadixTree::stamp_to_root(Node* n) {
  for (Node* p = n; p != nullptr && p != &root_; p = p->parent) {
    p->last_access = clock_;
    p->hits++;
    p->prio = std::max(p->prio, cur_prio_);
  }
}

int RadixTree::set_policy(int32_t policy) {
  if (policy < RDX_EVICT_LRU || policy > RDX_EVICT_PRIORITY)
    return fail(RDX_EINVAL, "rdx_tree_set_policy: unknown policy %d", policy);
  policy_ = policy;
  return ok();
}

int RadixTree::check_private(const int32_t* slots, int64_t n) {
  int rc = RDX_OK;
  int64_t i = 0;
  for (; i < n; ++i) {
    int32_t s = slots[i];
    if (s < 0 || s >= num_slots_) {
      rc = fail(RDX_EINVAL, "slot %d out of range [0, %lld)", s, (long long)num_slots_);
      break;
    }
    if (state_[s] != kPrivate) {
      rc = fail(RDX_ESTATE, "slot %d is not a private allocated slot (or is listed twice)", s);
      break;
    }
    state_[s] = 3;  // mark seen: a repeat fails the check above
  }
  for (int64_t j = 0; j < i; ++j) state_[slots[j]] = kPrivate;
  return rc;
}

int RadixTree::match_prefix(const int32_t* tokens, int64_t n, int32_t* out_slots, int64_t* out_len,
                            int64_t* out_node) {
  if (n < 0 || (n > 0 && (!tokens || !out_slots)) || !out_len || !out_node)
    return fail(RDX_EINVAL, "rdx_match_prefix: bad arguments");
  std::vector<WalkStep> steps;
  clock_++;
  int64_t m = walk(tokens, n, &steps);
  int64_t mu = (m / unit_) * unit_;
  *out_len = mu;
  if (mu == 0) {
    *out_node = 0;
    return ok();
  }
  int64_t pos = 0;
  for (const WalkStep& s : steps) {
    int64_t cnt = std::min<int64_t>(s.matched, mu - pos);
    std::copy(s.node->slots.begin(), s.node->slots.begin() + cnt, out_slots + pos);
    pos += cnt;
    if (pos == mu) break;
  }
  Node* e = node_ending_at(steps, mu);
  stamp_to_root(e);
  *out_node = e->id;
  return ok();
}

int RadixTree::lock(int64_t id) {
  const Node* c = find(id);
  if (!c) return fail(RDX_ESTATE, "rdx_lock: unknown node %lld", (long long)id);
  for (Node* p = const_cast<Node*>(c); p != &root_; p = p->parent) p->ref++;
  return ok();
}

int RadixTree::unlock(int64_t id) {
  const Node* c = find(id);
  if (!c) return fail(RDX_ESTATE, "rdx_unlock: unknown node %lld", (long long)id);
  for (const Node* p = c; p != &root_; p = p->parent)
    if (p->ref < 1) return fail(RDX_ESTATE, "rdx_unlock: reference count underflow at node %lld", (long long)p->id);
  for (Node* p = const_cast<Node*>(c); p != &root_; p = p->parent) p->ref--;
  return ok();
}

int64_t RadixTree::evict_until(int64_t free_target, int64_t min_freed) {
  using Key = std::tuple<int64_t, int64_t, int64_t, Node*>;
  std::priority_queue<Key, std::vector<Key>, std::greater<Key>> leaves;
  auto major = [this](const Node* x) -> int64_t {
    switch (policy_) {
      case RDX_EVICT_LFU: return x->hits;
      case RDX_EVICT_SLRU: return x->hits >= 2 ? 1 : 0;
      case RDX_EVICT_PRIORITY: return x->prio;
      default: return 0;
    }
  };
  for (auto& kv : nodes_) {
    Node* x = kv.second.get();
    if (x->ref == 0 && x->children.empty()) leaves.emplace(major(x), x->last_access, x->id, x);
  }
  int64_t freed = 0;
  while ((num_free() < free_target || freed < min_freed) && !leaves.empty()) {
    Node* v = std::get<3>(leaves.top());
    leaves.pop();
    Node* parent = v->parent;
    parent->children.erase(v->key[0]);
    for (int32_t s : v->slots) {
      state_[s] = kFree;
      release(s);
    }
    freed += (int64_t)v->key.size();
    evictions_++;
    nodes_.erase(v->id);
    if (parent != &root_ && parent->children.empty() && parent->ref == 0)
      leaves.emplace(major(parent), parent->last_access, parent->id, parent);
  }
  return freed;
}

int RadixTree::alloc(int64_t n, int32_t* out) {
  if (n < 0 || (n > 0 && !out)) return fail(RDX_EINVAL, "rdx_alloc: bad arguments");
  int64_t short_by = n - num_free();
  if (short_by > 0) {
    if (evictable_tokens() < short_by)
      return fail(RDX_ENOSPC, "rdx_alloc: need %lld slots, %lld free, %lld evictable", (long long)n,
                  (long long)num_free(), (long long)evictable_tokens());
    evict_until(n, 0);
    if (num_free() < n) return fail(RDX_ESTATE, "rdx_alloc: eviction fell short (inconsistent reference counts)");
  }
  // the n smallest free ids, ascending
  int64_t i = 0, w = low_word_;
  while (i < n) {
    uint64_t bits = free_bits_[w];
    while (bits && i < n) {
      const int b = __builtin_ctzll(bits);
      bits &= bits - 1;
      const int32_t s = (int32_t)(w * 64 + b);
      state_[s] = kPrivate;
      out[i++] = s;
    }
    free_bits_[w] = bits;
    if (!bits) ++w;
  }
  low_word_ = w;
  n_free_ -= n;
  return ok();
}

int RadixTree::free_slots(const int32_t* slots, int64_t n) {
  if (n < 0 || (n > 0 && !slots)) return fail(RDX_EINVAL, "rdx_free: bad arguments");
  int rc = check_private(slots, n);
  if (rc) return rc;
  for (int64_t i = 0; i < n; ++i) {
    state_[slots[i]] = kFree;
    release(slots[i]);
  }
  return ok();
}

int RadixTree::insert(const int32_t* tokens, const int32_t* slots, int64_t n, int64_t* out_present,
                      int64_t* out_node) {
  if (n < 0 || (n > 0 && (!tokens || !slots)) || !out_present || !out_node)
    return fail(RDX_EINVAL, "rdx_insert: bad arguments");
  std::vector<WalkStep> steps;
  int64_t k = walk(tokens, n, &steps);
  int rc = check_private(slots + k, n - k);
  if (rc) return rc;
  clock_++;
  Node* attach = k > 0 ? node_ending_at(steps, k) : &root_;
  *out_present = k;
  if (k == n) {
    stamp_to_root(attach);
    *out_node = attach == &root_ ? 0 : attach->id;
    return ok();
  }
  auto z = std::make_unique<Node>();
  z->id = next_id_++;
  z->parent = attach;
  z->start = k;
  z->key.assign(tokens + k, tokens + n);
  z->slots.assign(slots + k, slots + n);
  z->last_access = clock_;
  z->prio = cur_prio_;
  for (int64_t i = k; i < n; ++i) state_[slots[i]] = kTree;
  attach->children[tokens[k]] = z.get();
  stamp_to_root(attach);
  *out_node = z->id;
  nodes_[z->id] = std::move(z);
  return ok();
}

int RadixTree::evict(int64_t n_tokens, int64_t* out_freed) {
  if (!out_freed) return fail(RDX_EINVAL, "rdx_evict: bad arguments");
  *out_freed = n_tokens > 0 ? evict_until(0, n_tokens) : 0;
  return ok();
}

}  // namespace rdx
