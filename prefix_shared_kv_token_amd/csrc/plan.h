// Batch planner: turns a batch of requests (their locked tree nodes and page
// table rows) into the work list of one prefix-shared attention launch.
//
// Follows the BatchLLM explainer, Horizontal Fusion section: a request
// attends to the common-prefix KV and to its own KV; the two parts are
// computed by different workgroups of ONE kernel with tiles sized per part,
// and their partial results are combined.  Here a part is a "job": a key
// range of one page-table row, visible to a token range of a row tile.
#pragma once

#include <cstdint>
#include <vector>

#include "rdx.h"
#include "radix_tree.h"

namespace rdx {

constexpr int kTileRows = 128;   // query rows (token x grouped head) per tile
constexpr int kKeyBlock = 64;    // keys per inner iteration of the kernels
constexpr int kDecodeTileRows = 64;  // query rows per tile of the bf16 decode kernel

// Record layouts (int32 words) -- shared with the device code.
// item: one per key chunk, run for every KV head.  Words 0-3: tile,
// job_begin, job_end, contrib (index within the tile); 4: 64-key blocks of
// the item; 5-7: the tile's tok_begin, n_tok, split index (-1: none); 8-10:
// the contribution's tok_lo, tok_hi, ws_token_base (0, n_tok, 0 unsplit);
// 11-16: the first job (page_row, key_begin, key_end, tok_lo, tok_hi,
// causal); 17: the caller Q row of the tile's first token when the tile's
// rows are consecutive, else -1 -- everything a workgroup needs to start
// loading in one read.
constexpr int kItemWords = 20;
constexpr int kTileWords = 8;     // tok_begin, n_tok, n_contrib, contrib_begin, split index (-1: none), cptr base
constexpr int kJobWords = 8;      // page_row, key_begin, key_end, tok_lo, tok_hi, causal
constexpr int kTokWords = 2;      // q_index, position
constexpr int kContribWords = 4;  // tok_lo, tok_hi, ws_token_base
constexpr int kRunWords = 4;      // page_row, pos_begin, count, src_offset
constexpr int kMergeRows = 16;    // query rows per merge workgroup (16 lanes per row)
// merge block: first row, tile n_tok, tile tok_begin, first tile token t0 of
// the block, then the merge-list offsets (cptr) of tile tokens t0 .. t0+16
// (clamped to the tile's n_tok), padding
constexpr int kMBlockWords = 24;

struct Plan {
  rdx_attn_desc desc{};
  int32_t kind = 0;
  int32_t target_items = 0;
  int64_t ld = 0;
  // host records
  // merge of split tiles: per tile token, the partial states covering it
  // (cptr: n_tok + 1 offsets per split tile, tile word 5 = its base; clist:
  // the workspace token of each partial), and 16-row merge blocks carrying
  // the tile fields the merge needs (kMBlockWords)
  std::vector<int32_t> items, tiles, jobs, toks, contribs, runs, run_slots, new_slots, cptr, clist, mblocks;
  int64_t num_split_tiles = 0, num_shared_segments = 0, ws_tokens = 0, key_rows = 0;
  int64_t max_page_row = -1;
  // device blob layout, in int32 words
  int64_t off_items = 0, off_tiles = 0, off_jobs = 0, off_toks = 0, off_contribs = 0,
          off_runs = 0, off_run_slots = 0, off_new = 0, off_cptr = 0, off_clist = 0, off_mblocks = 0,
          total_words = 0;
  int64_t ws_ml_offset = 0, ws_bytes = 0;
  bool built = false;
  // upload staging, owned by the plan: a ring of pinned host buffers, each
  // with the event of the last copy out of it, so the host can prepare the
  // next uploads while earlier ones are still queued.  Decode plans keep 32
  // steps queued (a few hundred KB of lists): enough device work to cover
  // the host's completion and admission work between batches; extend plans
  // (lists of megabytes) keep 8.
  static constexpr int kMaxStages = 32;
  int n_stages = 8;
  struct Stage {
    void* pinned = nullptr;
    void* pinned_dev = nullptr;  // the same memory as the device addresses it
    int64_t bytes = 0;
    void* event = nullptr;
    bool pending = false;
  } stages[kMaxStages];
  int64_t uploads = 0;
  std::vector<void*> retired;  // outgrown staging buffers, freed with the plan

  // query rows per tile: 256 for the wide bf16 head_dim-128 extend kernel,
  // kDecodeTileRows for the bf16 decode kernel, kTileRows otherwise
  int tile_rows = kTileRows;
  int group() const { return desc.num_q_heads / desc.num_kv_heads; }
  int tile_tokens() const { return tile_rows / group(); }
  int build(const RadixTree& tree, const rdx_batch& b, int64_t ld);
  void layout();
  void fill_info(rdx_plan_info* out) const;
};

}  // namespace rdx
