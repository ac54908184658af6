// Edge-compressed radix tree over token ids, page size 1 (one KV slot per
// token), with reference counts and LRU leaf eviction, plus the KV slot
// allocator that shares the pool with running requests.
//
// Follows: SGLang explainer, RadixAttention section (prefix match, insert
// with split, recursive LRU leaf eviction of unreferenced nodes); SGLang
// paper notes, section 3 / Figure 3 (reference counts, the pool shared with
// running requests, splits when a new session shares part of an edge).
#pragma once

#include <cstdint>
#include <cstring>
#include <memory>
#include <queue>
#include <unordered_map>
#include <vector>

#include "rdx.h"

namespace rdx {

// Length of the common prefix of a[0..n) and b[0..n): equal 16-token blocks
// are skipped with memcmp, the first unequal block is scanned.
inline int64_t common_prefix(const int32_t* a, const int32_t* b, int64_t n) {
  constexpr int64_t kBlock = 16;
  int64_t i = 0;
  while (i + kBlock <= n && std::memcmp(a + i, b + i, kBlock * sizeof(int32_t)) == 0) i += kBlock;
  while (i < n && a[i] == b[i]) ++i;
  return i;
}

struct Node {
  int64_t id = 0;
  Node* parent = nullptr;
  int64_t start = 0;                 // position of key[0] in the sequence
  std::vector<int32_t> key;          // edge tokens
  std::vector<int32_t> slots;        // their KV slots
  std::unordered_map<int32_t, Node*> children;  // first token -> child
  int64_t last_access = 0;
  int64_t ref = 0;
  int64_t hits = 1;   // match/insert calls that stamped it (LFU, SLRU)
  int32_t prio = 0;   // highest priority of those calls (priority eviction)
  int64_t end() const { return start + (int64_t)key.size(); }
  // batch-planner scratch: meaningful only while plan_epoch equals the epoch
  // of the build that is running (builds on one tree are never concurrent)
  mutable int64_t plan_epoch = 0;
  mutable int32_t plan_count = 0;  // requests of the batch whose path holds this node
  mutable int32_t plan_seg = -1;   // shared segment starting at this node
};

class RadixTree {
 public:
  RadixTree(int64_t num_slots, int32_t match_unit);
  ~RadixTree();

  int match_prefix(const int32_t* tokens, int64_t n, int32_t* out_slots, int64_t* out_len,
                   int64_t* out_node);
  // Matched length rounded down to the matching unit, leaving the tree as it
  // is (no split, no clock tick): what ordering decisions look at.
  int64_t peek_match(const int32_t* tokens, int64_t n) const;
  int lock(int64_t node);
  int unlock(int64_t node);
  int alloc(int64_t n, int32_t* out);
  int free_slots(const int32_t* slots, int64_t n);
  int insert(const int32_t* tokens, const int32_t* slots, int64_t n, int64_t* out_present,
             int64_t* out_node);
  int evict(int64_t n_tokens, int64_t* out_freed);
  // eviction order among unreferenced leaves (RDX_EVICT_*) and the priority
  // the following match/insert calls carry
  int set_policy(int32_t policy);
  void set_priority(int32_t p) { cur_prio_ = p; }
  int32_t policy() const { return policy_; }

  int32_t match_unit() const { return unit_; }
  int64_t num_slots() const { return num_slots_; }
  int64_t num_free() const { return n_free_; }
  int64_t num_nodes() const { return (int64_t)nodes_.size(); }
  int64_t evictions() const { return evictions_; }
  int64_t clock() const { return clock_; }
  int64_t count_state(uint8_t s) const;
  int64_t evictable_tokens() const;

  // node lookup: nullptr if unknown; id 0 is the root
  const Node* find(int64_t id) const;
  const Node* root() const { return &root_; }

  static constexpr uint8_t kFree = 0, kTree = 1, kPrivate = 2;

 private:
  struct WalkStep {
    Node* node;
    int64_t matched;  // tokens of node->key matched
  };
  // Walks from the root; returns the matched length and the visited nodes.
  int64_t walk(const int32_t* tokens, int64_t n, std::vector<WalkStep>* steps);
  // Returns the node that ends exactly at depth d along the walked steps,
  // splitting the node containing d if needed.  d > 0.
  Node* node_ending_at(const std::vector<WalkStep>& steps, int64_t d);
  Node* split(Node* x, int64_t c);
  void stamp_to_root(Node* n);
  int64_t evict_until(int64_t free_target, int64_t min_freed);
  int check_private(const int32_t* slots, int64_t n);

  int64_t num_slots_;
  int32_t unit_;
  int32_t policy_ = RDX_EVICT_LRU;
  int32_t cur_prio_ = 0;
  Node root_;
  std::unordered_map<int64_t, std::unique_ptr<Node>> nodes_;
  int64_t next_id_ = 1;
  int64_t clock_ = 0;
  int64_t evictions_ = 0;
  std::vector<uint8_t> state_;
  // free set as a bitmap (bit s set <=> slot s free); every word below
  // low_word_ is fully allocated, so the smallest free ids are found by a
  // forward scan from there
  std::vector<uint64_t> free_bits_;
  int64_t n_free_ = 0;
  int64_t low_word_ = 0;
  void release(int32_t s) {
    free_bits_[s >> 6] |= uint64_t(1) << (s & 63);
    n_free_++;
    if ((s >> 6) < low_word_) low_word_ = s >> 6;
  }
};

}  // namespace rdx

// The C ABI's opaque tree handle.
struct rdx_tree {
  rdx::RadixTree impl;
  rdx_tree(int64_t n, int32_t u) : impl(n, u) {}
};
