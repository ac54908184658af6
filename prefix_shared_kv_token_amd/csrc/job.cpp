// Host side of the native token-batched job (rdx_job_*): per iteration the
// batcher's entries, admissions (match, lock, allocate the prompt's slots
// into the job's host page-table row), one allocation for the decode tokens,
// the plan over the mixed batch; after the launch, the requests that
// completed go into the tree (insert, free duplicates, unlock) and give their
// rows back.  The device part (upload, KV scatter, attention) is
// rdx_job_launch in device.hip.
#include "job.h"

#include <algorithm>
#include <new>

#include "common.h"

using rdx::fail;

namespace {

int broken(rdx_job* j, int rc) {
  j->broken = true;
  return rc;
}

}  // namespace

extern "C" {

int rdx_job_create(rdx_tree* tree, int32_t num_groups, const int32_t* prefix_len, const int32_t* member_offsets,
                   const int32_t* distinct_len, const int32_t* decode_len, int32_t s_chunk, int64_t m_threshold,
                   const int32_t* tokens, const int64_t* offsets, int32_t num_rows, int64_t ld, int32_t flags,
                   rdx_job** out) {
  if (!tree || !out || num_groups < 0 || !prefix_len || !member_offsets || num_rows <= 0 || ld <= 0 || !offsets)
    return fail(RDX_EINVAL, "rdx_job_create: bad arguments");
  const int32_t G = num_groups, M = member_offsets[num_groups];
  rdx_batcher* b = nullptr;
  int rc = rdx_batcher_create(G, prefix_len, member_offsets, distinct_len, decode_len, s_chunk, m_threshold, &b);
  if (rc) return rc;
  const int64_t n_tok = offsets[G + M] - offsets[0];
  if (offsets[0] != 0 || (n_tok > 0 && !tokens)) {
    rdx_batcher_destroy(b);
    return fail(RDX_EINVAL, "rdx_job_create: offsets must start at 0, tokens non-null");
  }
  // sequence lengths: prefix requests = their prefix; members = prefix +
  // distinct prompt + generated tokens
  for (int32_t g = 0; g < G; ++g) {
    const int64_t want = prefix_len[g];
    if (offsets[g + 1] - offsets[g] != want) {
      rdx_batcher_destroy(b);
      return fail(RDX_EINVAL, "rdx_job_create: group %d: prefix sequence of %lld tokens, expected %lld", g,
                  (long long)(offsets[g + 1] - offsets[g]), (long long)want);
    }
    for (int32_t m = member_offsets[g]; m < member_offsets[g + 1]; ++m) {
      const int64_t len = offsets[G + m + 1] - offsets[G + m];
      const int64_t w = (int64_t)prefix_len[g] + distinct_len[m] + decode_len[m];
      if (len != w || len > ld) {
        rdx_batcher_destroy(b);
        return fail(RDX_EINVAL, "rdx_job_create: member %d: sequence of %lld tokens, expected %lld (ld %lld)", m,
                    (long long)len, (long long)w, (long long)ld);
      }
    }
  }
  rdx_job* j;
  try {
    j = new rdx_job();
    j->tree = tree;
    j->batcher = b;
    j->G = G;
    j->M = M;
    j->tokens = tokens;
    j->offsets = offsets;
    j->prompt_len.resize(G + M);
    for (int32_t g = 0; g < G; ++g) {
      j->prompt_len[g] = prefix_len[g];
      for (int32_t m = member_offsets[g]; m < member_offsets[g + 1]; ++m)
        j->prompt_len[G + m] = (int64_t)prefix_len[g] + distinct_len[m];
    }
    j->ld = ld;
    j->num_rows = num_rows;
    j->host_pt.reset(new int32_t[(size_t)num_rows * ld]);
    j->row_kv.assign(num_rows, 0);
    j->row_written.assign(num_rows, 0);
    for (int32_t r = num_rows - 1; r >= 0; --r) j->free_rows.push_back(r);
    j->req_row.assign(G + M, -1);
    j->req_node.assign(G + M, 0);
    j->req_matched.assign(G + M, 0);
    j->keep_rows = (flags & RDX_JOB_KEEP_ROWS) != 0;
    j->dry_run = (flags & RDX_JOB_DRY_RUN) != 0;
    if (j->keep_rows) j->final_rows.resize(G + M);
    j->entries.resize((size_t)G + M + 1);
  } catch (const std::bad_alloc&) {
    rdx_batcher_destroy(b);
    return fail(RDX_EINVAL, "rdx_job_create: out of host memory");
  }
  *out = j;
  return rdx::ok();
}

void rdx_job_destroy(rdx_job* j) {
  if (!j) return;
  rdx_batcher_destroy(j->batcher);
  delete j;
}

int rdx_job_prepare(rdx_job* j, rdx_plan* extend_plan, rdx_plan* decode_plan, int64_t* out_tokens,
                    int32_t* out_kind, rdx_plan_info* out_info) {
  if (!j || !extend_plan || !decode_plan || !out_tokens) return fail(RDX_EINVAL, "rdx_job_prepare: bad arguments");
  if (j->broken) return fail(RDX_ESTATE, "rdx_job_prepare: an earlier error left the job inconsistent");
  if (j->state != 0) return fail(RDX_ESTATE, "rdx_job_prepare: the previous iteration is not complete");
  *out_tokens = 0;
  int32_t n = 0;
  int rc = rdx_batcher_next(j->batcher, j->entries.data(), (int32_t)j->entries.size(), &n);
  if (rc) return broken(j, rc);
  j->n_entries = n;
  if (n == 0) return rdx::ok();  // the job is done
  rdx::RadixTree& t = j->tree->impl;
  const int32_t G = j->G;
  auto req_of = [&](const rdx_tb_entry& e) { return e.kind == RDX_TB_PREFIX ? e.group : G + e.member; };
  // admissions, in entry order
  for (int32_t i = 0; i < n; ++i) {
    const rdx_tb_entry& e = j->entries[i];
    const int32_t r = req_of(e);
    if (j->req_row[r] >= 0) continue;
    if (e.kind == RDX_TB_DECODE) return broken(j, fail(RDX_ESTATE, "rdx_job_prepare: decode of an unadmitted request"));
    if (j->free_rows.empty()) return broken(j, fail(RDX_ENOSPC, "rdx_job_prepare: no free page-table row"));
    const int32_t row = j->free_rows.back();
    j->free_rows.pop_back();
    int32_t* pt = j->host_pt.get() + (int64_t)row * j->ld;
    const int64_t len = j->prompt_len[r];
    int64_t m = 0, node = 0;
    rc = t.match_prefix(j->tokens + j->offsets[r], len, pt, &m, &node);
    if (rc) return broken(j, rc);
    rc = t.lock(node);
    if (rc) return broken(j, rc);
    rc = t.alloc(len - m, pt + m);
    if (rc) return broken(j, rc);
    j->req_row[r] = row;
    j->req_node[r] = node;
    j->req_matched[r] = m;
    j->row_kv[row] = (int32_t)len;
    j->row_written[row] = 0;
  }
  // one allocation for the decode tokens (decode entries come first)
  int32_t n_dec = 0;
  while (n_dec < n && j->entries[n_dec].kind == RDX_TB_DECODE) ++n_dec;
  j->b_node.resize(n);
  j->b_row.resize(n);
  j->b_kv.resize(n);
  j->b_q.resize(n);
  j->b_wr.resize(n);
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) total += j->entries[i].count;
  j->b_new.resize(std::max<int64_t>(total, 1));
  if (n_dec > 0) {
    rc = t.alloc(n_dec, j->b_new.data());
    if (rc) return broken(j, rc);
  }
  int64_t w = n_dec;
  for (int32_t i = 0; i < n; ++i) {
    const rdx_tb_entry& e = j->entries[i];
    const int32_t r = req_of(e), row = j->req_row[r];
    int32_t* pt = j->host_pt.get() + (int64_t)row * j->ld;
    const int64_t end = (int64_t)e.begin + e.count;
    if (end > j->ld) return broken(j, fail(RDX_EINVAL, "rdx_job_prepare: request %d beyond ld", r));
    if (e.kind == RDX_TB_DECODE) {
      pt[e.begin] = j->b_new[i];
    } else {
      std::copy(pt + e.begin, pt + end, j->b_new.data() + w);
      w += e.count;
    }
    j->b_node[i] = j->req_node[r];
    j->b_row[i] = row;
    j->b_kv[i] = (int32_t)end;
    j->b_q[i] = e.count;
    j->b_wr[i] = j->row_written[row];
    j->row_kv[row] = (int32_t)end;
  }
  j->kind = n_dec == n ? RDX_PLAN_DECODE : RDX_PLAN_EXTEND;
  j->plan = reinterpret_cast<rdx::Plan*>(j->kind == RDX_PLAN_DECODE ? decode_plan : extend_plan);
  if (j->plan->kind != j->kind) return broken(j, fail(RDX_EINVAL, "rdx_job_prepare: plan kinds swapped"));
  rdx_batch bt{n, 0, j->b_node.data(), j->b_row.data(), j->b_kv.data(), j->b_q.data(), j->b_wr.data(),
               j->b_new.data()};
  j->plan->ld = j->ld;
  rc = j->plan->build(t, bt, j->ld);
  if (rc) return broken(j, rc);
  if (out_info) j->plan->fill_info(out_info);
  if (out_kind) *out_kind = j->kind;
  j->n_tokens = total;
  *out_tokens = total;
  j->state = 1;
  return rdx::ok();
}

int rdx_job_complete(rdx_job* j, int32_t* out_finished) {
  if (!j) return fail(RDX_EINVAL, "rdx_job_complete: bad arguments");
  if (j->broken) return fail(RDX_ESTATE, "rdx_job_complete: an earlier error left the job inconsistent");
  if (j->state != 2 && !(j->dry_run && j->state == 1))
    return fail(RDX_ESTATE, "rdx_job_complete: the iteration was not launched");
  rdx::RadixTree& t = j->tree->impl;
  const int32_t G = j->G;
  int32_t fin = 0;
  for (int32_t i = 0; i < j->n_entries; ++i) {
    const rdx_tb_entry& e = j->entries[i];
    const int32_t r = e.kind == RDX_TB_PREFIX ? e.group : G + e.member;
    const int32_t row = j->req_row[r];
    j->row_written[row] = j->b_kv[i];
    const int64_t len = j->offsets[r + 1] - j->offsets[r];
    if ((int64_t)e.begin + e.count != len) continue;
    int32_t* pt = j->host_pt.get() + (int64_t)row * j->ld;
    int64_t present = 0, nd = 0;
    int rc = t.insert(j->tokens + j->offsets[r], pt, len, &present, &nd);
    if (rc) return broken(j, rc);
    const int64_t m = j->req_matched[r];
    if (present > m) {
      rc = t.free_slots(pt + m, present - m);
      if (rc) return broken(j, rc);
    }
    rc = t.unlock(j->req_node[r]);
    if (rc) return broken(j, rc);
    if (j->keep_rows) j->final_rows[r].assign(pt, pt + len);
    j->req_row[r] = -2;  // finished
    j->free_rows.push_back(row);
    ++fin;
  }
  if (out_finished) *out_finished = fin;
  j->state = 0;
  return rdx::ok();
}

int rdx_job_row(const rdx_job* j, int32_t req, int32_t* out, int64_t cap, int64_t* out_len, int64_t* out_matched) {
  if (!j || !out_len || req < 0 || req >= j->G + j->M) return fail(RDX_EINVAL, "rdx_job_row: bad arguments");
  if (!j->keep_rows) return fail(RDX_ESTATE, "rdx_job_row: the job keeps no rows");
  const std::vector<int32_t>& r = j->final_rows[req];
  *out_len = (int64_t)r.size();
  if (out_matched) *out_matched = j->req_matched[req];
  if (cap < (int64_t)r.size()) return fail(RDX_ENOBUFS, "rdx_job_row: %lld entries", (long long)r.size());
  if (!r.empty()) std::copy(r.begin(), r.end(), out);
  return rdx::ok();
}

}  // extern "C"
