// A token-batched job (BatchLLM explainer: Throughput-oriented and
// Memory-centric Token Batching, Horizontal Fusion) run natively, one
// iteration per prepare / launch / complete triple; see rdx_job_* in rdx.h.
#pragma once

#include <cstdint>
#include <memory>
#include <vector>

#include "plan.h"
#include "radix_tree.h"
#include "rdx.h"

struct rdx_job {
  rdx_tree* tree = nullptr;    // borrowed
  rdx_batcher* batcher = nullptr;  // owned
  int32_t G = 0, M = 0;        // groups; members (request G + m)
  const int32_t* tokens = nullptr;  // every request's full sequence (the caller's)
  const int64_t* offsets = nullptr;
  std::vector<int64_t> prompt_len;
  int64_t ld = 0;
  int32_t num_rows = 0;
  std::unique_ptr<int32_t[]> host_pt;  // num_rows x ld, written before read
  std::vector<int32_t> row_kv, row_written, free_rows;
  std::vector<int32_t> req_row;
  std::vector<int64_t> req_node, req_matched;
  bool keep_rows = false;
  bool dry_run = false;        // iterations complete without a launch (host planning)
  std::vector<std::vector<int32_t>> final_rows;
  // the prepared iteration
  std::vector<rdx_tb_entry> entries;
  int32_t n_entries = 0;
  std::vector<int64_t> b_node;
  std::vector<int32_t> b_row, b_kv, b_q, b_wr, b_new;
  rdx::Plan* plan = nullptr;   // the plan built for it (borrowed)
  int32_t kind = 0;
  int64_t n_tokens = 0;
  int state = 0;               // 0 idle, 1 prepared, 2 launched
  bool broken = false;         // an error left the job inconsistent
};
