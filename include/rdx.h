/*
 * rdx.h -- C ABI of librdx: prefix-shared attention over a token-granular
 * paged KV pool whose prefixes are shared through a radix tree.
 *
 * Operations and the passages that define them:
 *   radix tree (match / insert / lock / LRU leaf eviction, page size 1):
 *     SGLang explainer (0h-n0.github.io ... paper-2312-07104-scheduling),
 *     RadixAttention section; SGLang paper notes (knowledge.zhaoweiguo.com
 *     ... 2312.07104_sglang), section 3 and Figure 3.
 *   matching unit (a match counted in whole units of u tokens):
 *     vLLM-vs-SGLang prefix caching page (zvxbase.com), worked example and
 *     matching-unit section.
 *   prefix-shared attention with horizontal fusion (shared-prefix part and
 *     distinct part in one launch, partial softmax states combined):
 *     BatchLLM explainer (0h-n0.github.io ... paper-2412-03594), Horizontal
 *     Fusion section.
 *   decode over prefix + distinct pages: same page, prefix-shared attention;
 *     vLLM-vs-SGLang page, section on prefill vs decode.
 *
 * Conventions
 *   - Every function returns RDX_OK (0) or a negative RDX_E* code; after an
 *     error rdx_last_error() describes it (thread-local, valid until the next
 *     rdx call on the thread).  A failed call leaves all state unchanged.
 *   - Slots (= pages = one token's KV row) are int32 in [0, num_slots).
 *   - Host pointers are caller-owned; output buffers must hold the stated
 *     capacity.  Device pointers are caller-owned device memory; the library
 *     never allocates or frees device memory (it allocates pinned host
 *     staging memory for plan uploads).
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Device calls only enqueue work; they do not synchronise, except where
 *     stated: a plan upload (and the decode step and job launch that make
 *     one) waits while the pinned staging buffer it reuses is still being
 *     read, and rdx_timing_read waits for the launches it reports.  Faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - Not thread-safe per object: one thread drives a tree and its plans.
 */
#ifndef RDX_H
#define RDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RDX_OK 0
#define RDX_EINVAL (-1)       /* bad argument */
#define RDX_ENOSPC (-2)       /* free + evictable slots < requested */
#define RDX_ESTATE (-3)       /* unknown node, refcount underflow, slot not private */
#define RDX_EUNSUPPORTED (-4) /* dtype / head_dim / head ratio not built */
#define RDX_EDEVICE (-5)      /* a HIP call failed */
#define RDX_ENOBUFS (-6)      /* a caller buffer is too small (sizes reported) */

const char* rdx_last_error(void);
const char* rdx_version(void);

/* ------------------------------------------------------------------ tree */
typedef struct rdx_tree rdx_tree;

/* A radix tree over token ids whose values are KV slots, page size 1.
 * num_slots: size of the KV pool (slots 0..num_slots-1 start free).
 * match_unit: rdx_match_prefix reports matches rounded down to a multiple of
 * it (1 = token-granular).  Errors: EINVAL (num_slots <= 0 or >= 2^31,
 * match_unit < 1). */
int rdx_tree_create(int64_t num_slots, int32_t match_unit, rdx_tree** out);
void rdx_tree_destroy(rdx_tree* tree);

/* Longest cached prefix of tokens[0..n): *out_len = m (rounded to the match
 * unit), out_slots[0..m) = its slots (capacity n), *out_node = the node that
 * ends exactly at m (0 = root when m == 0).  A match ending inside an edge
 * splits the edge there.  Ticks the LRU clock and stamps every node on the
 * path (a split keeps the old stamp and id on its lower part; the new upper
 * part takes the next node id and the reference count).  Errors: EINVAL. */
int rdx_match_prefix(rdx_tree* tree, const int32_t* tokens, int64_t n,
                     int32_t* out_slots, int64_t* out_len, int64_t* out_node);

/* +1 / -1 on the reference count of every node from `node` up to the root.
 * Referenced nodes are never evicted.  Errors: ESTATE (unknown node,
 * underflow). node 0 (root) is a no-op. */
int rdx_lock(rdx_tree* tree, int64_t node);
int rdx_unlock(rdx_tree* tree, int64_t node);

/* The n smallest free slots, ascending, into out_slots (capacity n); they
 * become private to the caller.  If fewer than n are free, least recently
 * used unreferenced leaves are evicted (whole nodes, smallest (last access,
 * node id) first, repeating as parents become leaves) until n are free.
 * Errors: EINVAL (n < 0), ENOSPC (free + evictable < n; nothing changes). */
int rdx_alloc(rdx_tree* tree, int64_t n, int32_t* out_slots);

/* Return private slots to the free set.  Errors: EINVAL (out of range),
 * ESTATE (a slot not private, or listed twice). */
int rdx_free(rdx_tree* tree, const int32_t* slots, int64_t n);

/* Insert tokens[0..n) with their slots.  *out_present = k, the length already
 * cached (the tree keeps its own slots for [0,k); the caller frees its
 * duplicates in [matched, k)); slots[k..n) must be private and become the
 * tree's.  *out_node = the node ending at n (split if inside an edge).  Ticks
 * the clock and stamps the path.  Errors: EINVAL, ESTATE. */
int rdx_insert(rdx_tree* tree, const int32_t* tokens, const int32_t* slots, int64_t n,
               int64_t* out_present, int64_t* out_node);

/* Evict LRU unreferenced leaves until at least n_tokens were freed or none
 * is left; *out_freed = tokens freed (may exceed n_tokens). */
int rdx_evict(rdx_tree* tree, int64_t n_tokens, int64_t* out_freed);

/* Batch admission -- the serving loop's admit step for a whole batch in one
 * call, the same call sequence as doing it request by request (SGLang
 * explainer, RadixAttention section: match the prompt against the tree,
 * lock the matched path, allocate slots for the rest, evicting LRU leaves
 * when short).  Request i's prompt is tokens[offsets[i] .. offsets[i+1])
 * (length n_i <= ld) and it owns host page-table row rows[i] (< num_rows) of
 * host_page_table (host int32 [num_rows][ld]).  For i = 0, 1, ...:
 * rdx_match_prefix (its slots go to row[0..m_i)), rdx_lock of the matched
 * node, rdx_alloc(n_i - m_i) into row[m_i..n_i); out_matched[i] = m_i,
 * out_node[i] = the node, and the new slots are also appended to
 * out_new_slots (request-major; capacity offsets[num_reqs] - offsets[0]).
 * *out_admitted = the number of requests admitted.  On an error (EINVAL,
 * ENOSPC, ESTATE) at request i, requests 0..i-1 stay admitted (locked,
 * rows written), request i holds no lock and no slots, and the later
 * requests are untouched. */
int rdx_admit(rdx_tree* tree, int32_t num_reqs, const int32_t* tokens, const int64_t* offsets,
              const int32_t* rows, int32_t* host_page_table, int64_t num_rows, int64_t ld,
              int64_t* out_matched, int64_t* out_node, int32_t* out_new_slots, int32_t* out_admitted);

/* Batch completion (SGLang explainer, RadixAttention section: after a
 * request completes, its tokens are inserted so later requests can reuse
 * them), request by request: insert tokens[offsets[i] .. offsets[i+1])
 * (prompt + generated, n_i <= ld) with the slots of host page-table row
 * rows[i] positions 0..n_i-1; free the request's duplicates in
 * [matched[i], present) where present is the length the tree already held;
 * unlock node[i].  *out_done = the number of requests finished; on an error
 * (EINVAL, ESTATE) at request i the earlier ones stay finished and request i
 * is untouched. */
int rdx_finish(rdx_tree* tree, int32_t num_reqs, const int32_t* tokens, const int64_t* offsets,
               const int32_t* rows, const int32_t* host_page_table, int64_t num_rows, int64_t ld,
               const int64_t* matched, const int64_t* node, int32_t* out_done);

/* Cache-aware ordering of the waiting requests (SGLang paper notes,
 * section 3 "cache-aware scheduling" and appendix A.2; vLLM-vs-SGLang page,
 * cache-aware ordering).  Request i's prompt is tokens[offsets[i] ..
 * offsets[i+1]), requests listed in arrival order.  Writes a permutation of
 * 0..num_reqs-1 to out_order: greedily, the next request is the one whose
 * prompt shares the longest prefix with the tree or with a request already
 * placed ahead of it in this order (its tokens will be cached when the later
 * one runs); ties go to the earliest arrival; shared lengths count whole
 * matching units.  out_score[k] = that shared length of request out_order[k]
 * when it was placed.  With more than fcfs_above requests: arrival order and
 * zero scores, no matching (the queue-length cut-off of the vLLM-vs-SGLang
 * page; 128 there).  The tree is only read -- no split, no LRU stamp.
 * Errors: EINVAL (null array, negative count, decreasing offsets). */
int rdx_schedule(const rdx_tree* tree, int32_t num_reqs, const int32_t* tokens, const int64_t* offsets,
                 int32_t fcfs_above, int32_t* out_order, int64_t* out_score);

/* Throughput-oriented token batching (BatchLLM explainer: Throughput-oriented
 * Token Batching, Equations 3-4; three-queue fetching; Memory-centric Token
 * Batching).  A job of num_groups groups: group g has a common prefix of
 * prefix_len[g] >= 0 tokens and members member_offsets[g] ..
 * member_offsets[g+1]-1 (member_offsets[0] = 0, at least one member per
 * group); member m has a distinct prompt of distinct_len[m] >= 1 tokens and
 * generates decode_len[m] >= 0 tokens.  Groups run in descending
 * R_group = 1 / (prefix + sum of distinct prompts), ties by index.  Each
 * rdx_batcher_next call is one iteration: one DECODE entry per request
 * decoding (in group order, then member order), then prefill chunks of
 * min(s_chunk, remaining) tokens in queue order -- DISTINCT chunks of
 * members whose group prefix was completed in an earlier iteration, then
 * PREFIX chunks of groups not yet prefilled, one chunk per item -- stopping
 * at the first chunk that would take the memory above m_threshold; memory =
 * 2 x (the prefix of every group with a decoding request, once) + 2 x (each
 * decoding request's distinct prompt + tokens generated before this
 * iteration) + 2 x (chunk tokens taken).  A member decodes from
 * the iteration after its prompt completes; its t-th token sits at
 * position prefix + distinct + t.  Needs m_threshold >= 2 s_chunk (an
 * iteration with nothing decoding always takes a chunk).  The arrays are
 * copied; errors: EINVAL. */
#define RDX_TB_DECODE 0
#define RDX_TB_DISTINCT 1
#define RDX_TB_PREFIX 2
typedef struct rdx_batcher rdx_batcher;
typedef struct rdx_tb_entry {
  int32_t kind;   /* RDX_TB_DECODE, RDX_TB_DISTINCT or RDX_TB_PREFIX */
  int32_t group;  /* group index */
  int32_t member; /* member index (global), -1 for PREFIX */
  int32_t begin;  /* position of the first token in its sequence */
  int32_t count;  /* tokens (1 for DECODE) */
} rdx_tb_entry;
int rdx_batcher_create(int32_t num_groups, const int32_t* prefix_len, const int32_t* member_offsets,
                       const int32_t* distinct_len, const int32_t* decode_len, int32_t s_chunk,
                       int64_t m_threshold, rdx_batcher** out);
void rdx_batcher_destroy(rdx_batcher* batcher);
/* Next iteration's entries into out[0 .. *out_n) (decode entries first);
 * *out_n = 0 once every token of the job has been emitted.  If cap is too
 * small: RDX_ENOBUFS with *out_n = the entries needed and no state change
 * (members + groups entries always suffice). */
int rdx_batcher_next(rdx_batcher* batcher, rdx_tb_entry* out, int32_t cap, int32_t* out_n);

/* Eviction order among unreferenced leaves (vLLM-vs-SGLang page, eviction
 * passage: SGLang offers LFU, SLRU and priority besides the default LRU;
 * named only there, taken here in their textbook forms).  Every match or
 * insert call that stamps a node also counts one access to it and raises
 * its priority to the call's (rdx_tree_set_priority; 0 by default); a new
 * node starts with one access and the call's priority; a split's upper part
 * copies both.  Victim = smallest (major key, last access, node id):
 * LRU major 0; LFU major = accesses; SLRU major = 1 once accessed by two
 * calls (protected), else 0 (probation, evicted first); PRIORITY major =
 * priority.  Errors: EINVAL (unknown policy). */
#define RDX_EVICT_LRU 0
#define RDX_EVICT_LFU 1
#define RDX_EVICT_SLRU 2
#define RDX_EVICT_PRIORITY 3
int rdx_tree_set_policy(rdx_tree* tree, int32_t policy);
/* Priority carried by the tree's following match/insert calls. */
int rdx_tree_set_priority(rdx_tree* tree, int32_t priority);

/* Global prefix analysis (BatchLLM explainer, Global Prefix Sharing): group
 * the requests of a batch -- prompt i = tokens[offsets[i] .. offsets[i+1])
 * -- so that each group's members share the group's prefix (computed once)
 * and compute the rest of their prompt on their own, choosing the groups by
 * the dynamic program over the batch's radix tree that minimises
 *   N_processed = sum of group prefixes + sum of (prompt - group prefix)
 * (the explainer's gain (leaves(c') - 1) x tokens(c') against the penalty
 * tokens(c), applied at every node; Equation 2's N_processed).  Ties keep
 * the higher node: one group for everything below; a request alone below a
 * branch is grouped at the first token of its own edge.  out_group[i] =
 * group id (numbered by first request), out_prefix[i] = the group's prefix
 * length; *out_num_groups, *out_processed = N_processed.  The tree is built
 * from the sorted prompts, not from the cache.  Errors: EINVAL. */
int rdx_prefix_groups(int32_t num_reqs, const int32_t* tokens, const int64_t* offsets, int32_t* out_group,
                      int64_t* out_prefix, int32_t* out_num_groups, int64_t* out_processed);

typedef struct rdx_stats {
  int64_t num_slots;
  int64_t free;      /* slots in the free set */
  int64_t cached;    /* slots held by the tree */
  int64_t evictable; /* tree slots with reference count 0 */
  int64_t private_;  /* slots allocated to callers and not inserted */
  int64_t nodes;     /* nodes excluding the root */
  int64_t evictions; /* nodes evicted so far */
  int64_t clock;     /* LRU clock (match + insert calls) */
} rdx_stats;
int rdx_tree_stats(const rdx_tree* tree, rdx_stats* out);

typedef struct rdx_node_info {
  int64_t id, parent, start, length, ref, last_access, num_children, hits, priority;
} rdx_node_info;
/* Introspection of one node; out_slots (capacity info.length, may be NULL)
 * receives its slots.  Errors: ESTATE (unknown node). */
int rdx_node_get(const rdx_tree* tree, int64_t node, rdx_node_info* out, int32_t* out_slots);

/* ------------------------------------------------------------ attention */
#define RDX_F32 0
#define RDX_BF16 1

typedef struct rdx_attn_desc {
  int32_t dtype;        /* RDX_F32 or RDX_BF16: Q, the KV pools and O */
  int32_t num_q_heads;  /* Hq */
  int32_t num_kv_heads; /* Hkv, divides Hq; query head h reads KV head h*Hkv/Hq */
  int32_t head_dim;     /* 64 or 128 */
  float sm_scale;       /* 0 -> 1/sqrt(head_dim) */
  int32_t kv_row_pitch; /* elements from one slot's row to the next in each KV
                           pool: 0 = Hkv*head_dim (dense), else >= Hkv*head_dim
                           with pitch*element size a multiple of 16 bytes */
  int64_t num_slots;    /* rows of each KV pool */
} rdx_attn_desc;
/* Layouts (row-major):
 *   K pool, V pool   [num_slots][pitch] elements, slot s's [Hkv][head_dim]
 *                    at the start of row s (pitch = kv_row_pitch or dense)
 *   Q, O, new K/V    [tokens][H][head_dim]   (H = Hq for Q/O, Hkv for K/V)
 *   page table       int32 [rows][ld]: row r, position p -> slot  */

/* The row pitch the kernels stream fastest (elements; a caller allocates its
 * pools with it and stores it in kv_row_pitch).  Each workgroup reads one KV
 * head's slice of every row it visits; with a dense row of a multiple of
 * 1 KiB, some heads' slices fall on the same few memory channels for every
 * row and stream ~25 % slower than the others, so the rows are padded by
 * 256 bytes.  desc->kv_row_pitch is ignored.  Errors: EINVAL. */
int rdx_kv_row_pitch_recommended(const rdx_attn_desc* desc, int32_t* out);

/* Scatter new K/V rows into the pools: pool[slots[i]] = new[i], i < n.
 * The pages only say that each token's KV lives in GPU pages that requests
 * share (SGLang paper notes, section 3); this is the plumbing that puts it
 * there.  slots: device int32[n], distinct.  Errors: EINVAL, EUNSUPPORTED,
 * EDEVICE. */
int rdx_kv_store(const rdx_attn_desc* desc, void* k_pool, void* v_pool,
                 const void* k_new, const void* v_new, const int32_t* slots,
                 int64_t n, void* stream);

/* ------------------------------------------------------------------ plan */
/* The work list of one attention launch.  Its structure is this library's:
 * the BatchLLM explainer (Horizontal Fusion) has the shared-prefix part and
 * each request's distinct part computed by different workgroups of one
 * kernel and their partial results combined; here a part is a job (a key
 * range of one page-table row for a token range of a row tile), and a tile
 * whose key ranges are split across workgroups is combined by the merge. */
typedef struct rdx_plan rdx_plan;
#define RDX_PLAN_EXTEND 0
#define RDX_PLAN_DECODE 1

/* One batch of requests.  Request i owns page-table row row[i]; after this
 * batch its positions 0..kv_len[i]-1 hold KV; its q_len[i] newest positions
 * kv_len[i]-q_len[i] .. kv_len[i]-1 are the new tokens, which are also its
 * queries (caller Q rows sum(q_len[0..i)) .. +q_len[i]).  node[i] is the
 * locked tree node ending the request's cached prefix (its depth must not
 * exceed kv_len-q_len; 0 = nothing cached); nodes reached by two or more
 * requests of the batch are attended to once for all of them.  Positions
 * [0, written[i]) of the row already hold the right slots on the device; the
 * upload writes [written[i], kv_len[i]) from the tree path and new_slots
 * (request-major, sum(q_len) entries). */
typedef struct rdx_batch {
  int32_t num_reqs;
  int32_t reserved;
  const int64_t* node;
  const int32_t* row;
  const int32_t* kv_len;
  const int32_t* q_len;
  const int32_t* written;
  const int32_t* new_slots;
} rdx_batch;

/* kind: RDX_PLAN_EXTEND or RDX_PLAN_DECODE; target_items: the launch size
 * (workgroups = item records x Hkv) the planner splits key ranges towards;
 * 0 = the default for MI355X's 256 CUs: 256 for the 256-row extend kernel,
 * 512 for the others, 256 for decode launches whose items would each get 32
 * or more 64-key blocks that way.  When a launch has fewer tiles than the
 * target, the target's items are handed out to the tiles with the longest
 * pieces (never more than the target); when a launch runs more than one
 * round of tiles with a short last round, its last tiles are cut into
 * pieces of a quarter tile or less.  Errors: EINVAL, EUNSUPPORTED. */
int rdx_plan_create(const rdx_attn_desc* desc, int32_t kind, int32_t target_items, rdx_plan** out);
void rdx_plan_destroy(rdx_plan* plan);

/* Build the work list of one batch: requests are ordered depth-first by
 * their shared nodes, queries are packed into row tiles, each tile gets the
 * shared segments and per-request own ranges it must attend to, and long key
 * ranges are split into separate work items whose partial softmax states a
 * merge kernel combines, issued by the same attention call right behind it.
 * Extend tiles group the requests that share their deepest shared segment;
 * decode tiles group one top-level sharing group, and inside it a run of
 * requests sharing the next segment down starts a fresh tile when it would
 * overflow the current one but fits in one of its own (so such a segment is
 * streamed by one tile).  page_table_ld: row stride of the page table.
 * Errors: EINVAL (inconsistent batch), ESTATE (unknown node). */
int rdx_plan_build(rdx_plan* plan, const rdx_tree* tree, const rdx_batch* batch,
                   int64_t page_table_ld);

typedef struct rdx_plan_info {
  int64_t device_bytes;      /* size of the device plan buffer */
  int64_t workspace_bytes;   /* attention workspace (0 when nothing is split) */
  int64_t new_slots_offset;  /* byte offset of the new-token slot list (int32[num_new]) */
  int64_t num_new;           /* = sum(q_len) */
  int64_t num_items;         /* workgroups of the launch: item records x Hkv */
  int64_t num_tiles, num_jobs, num_split_tiles, num_shared_segments;
  int64_t key_rows;          /* sum over items of (tile rows x keys): work estimate */
} rdx_plan_info;
int rdx_plan_get_info(const rdx_plan* plan, rdx_plan_info* out);

/* Copy the plan to dev_plan (device, >= device_bytes) on `stream` and write
 * the batch's page-table entries into page_table (device int32
 * [page_table_rows][ld]).  The plan stages uploads through a ring of N
 * pinned host buffers (N = 32 for decode plans, 8 for extend plans), read by
 * a copy kernel through their device mapping (no DMA copy); the call blocks
 * only while the upload made N calls earlier has not left its buffer yet,
 * and grows the ring (pinned allocations) when a plan outgrows it.
 * Errors: EINVAL, EDEVICE. */
int rdx_plan_upload(rdx_plan* plan, void* dev_plan, int64_t dev_plan_bytes,
                    int32_t* page_table, int64_t page_table_rows, void* stream);

/* Host view of a built plan (for tests and tools).  Arrays stay valid until
 * the next rdx_plan_build.  Record layouts are int32:
 *   item    [20] tile, job_begin, job_end, contrib, then copies of what a
 *               workgroup needs first (block count, tile and contribution
 *               fields, first job) -- one per key chunk; the launch runs
 *               item i for KV head h as workgroup i * Hkv + h
 *   tile    [8] tok_begin, n_tok, n_contrib, contrib_begin, split index
 *               (-1 = not split), merge-list base, 0, 0
 *   job     [8] page_row, key_begin, key_end, tok_lo, tok_hi, causal, 0, 0
 *   token   [2] q_index, position
 *   contrib [4] tok_lo, tok_hi, ws_token_base, 0 */
typedef struct rdx_plan_view {
  const int32_t* items; int64_t num_items;
  const int32_t* tiles; int64_t num_tiles;
  const int32_t* jobs; int64_t num_jobs;
  const int32_t* tokens; int64_t num_tokens;
  const int32_t* contribs; int64_t num_contribs;
  int32_t tile_rows;       /* query rows per tile (tokens x Hq/Hkv) */
  int32_t group;           /* Hq / Hkv */
} rdx_plan_view;
int rdx_plan_get_view(const rdx_plan* plan, rdx_plan_view* out);

/* ------------------------------------------------------ attention launch */
/* Prefix-shared attention of one plan (extend or decode kind respectively):
 * for every new token at position p and query head h,
 *   O[tok][h] = softmax_j(scale * q.k_j) v_j  over positions j <= p of its row,
 * reading K/V through the page table.  Work items cover (row tile, KV head,
 * key ranges); a tile streams its shared-prefix keys and its requests' own
 * keys with one online-softmax state.  Tiles whose key ranges the planner
 * split over several items write partial (o, max, sum) states to the
 * workspace, and a merge kernel enqueued right behind combines them by
 * log-sum-exp.  q/o: device [sum q_len][Hq][head_dim] in caller order.
 * workspace: device scratch for the partial states, >= workspace_bytes, no
 * initial contents needed; may be NULL when workspace_bytes == 0.  Launches
 * sharing a workspace must be stream-ordered.  Errors: EINVAL, EUNSUPPORTED,
 * EDEVICE. */
int rdx_extend_attention(const rdx_attn_desc* desc, const rdx_plan* plan, const void* dev_plan,
                         const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_table, void* o, void* workspace,
                         int64_t workspace_bytes, void* stream);
int rdx_decode_attention(const rdx_attn_desc* desc, const rdx_plan* plan, const void* dev_plan,
                         const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_table, void* o, void* workspace,
                         int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): rdx_decode_attention
 * with no workspace argument.  The partial states of split tiles go to a
 * workspace built into the library: one 64 MiB device array per GPU, held
 * until the process ends (its address is looked up once per device, on the
 * first call with that device current).  Allocates nothing and calls no
 * allocating routine.  A plan whose split tiles need more than 64 MiB
 * (rdx_plan_get_info workspace_bytes) is rejected with EINVAL before
 * anything is enqueued.  Every call on one GPU uses the same array, and a
 * call's merge reads what its own attention kernel wrote there: calls that
 * overlap on one GPU (different streams, no ordering between them) race;
 * calls on one stream are ordered and safe.  Nothing in the array needs to
 * start at zero.  Other arguments, results and errors as for
 * rdx_decode_attention. */
int rdx_decode_attention_noalloc(const rdx_attn_desc* desc, const rdx_plan* plan, const void* dev_plan,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* page_table, void* o, void* stream);

/* ------------------------------------------------------- decode step */
/* Caller-owned device buffers of one step. */
typedef struct rdx_step_io {
  void* dev_plan;            /* device plan buffer and its size in bytes */
  int64_t dev_plan_bytes;
  void* workspace;           /* attention workspace and its size in bytes */
  int64_t workspace_bytes;
  int32_t* page_table;       /* device int32 [page_table_rows][ld] */
  int64_t page_table_rows;
  void* k_pool;              /* device [num_slots][pitch] each (desc->kv_row_pitch) */
  void* v_pool;
  const void* q;             /* device [num_reqs][Hq][head_dim] */
  const void* k_new;         /* device [num_reqs][Hkv][head_dim] each */
  const void* v_new;
  void* o;                   /* device [num_reqs][Hq][head_dim] */
} rdx_step_io;

/* One decode step of a running batch in one call -- the serving loop's
 * per-token path (SGLang explainer, RadixAttention section: slots come from
 * the pool the cache shares, the page table maps positions to slots; BatchLLM
 * explainer, Horizontal Fusion: shared prefixes are attended once per group).
 * Every request gets one new token:
 *   1. rdx_alloc(num_reqs) -> out_slots (slot i to request i);
 *   2. host_page_table[row[i]][row_kv_len[row[i]]] = out_slots[i] and
 *      row_kv_len[row[i]] += 1 (host arrays indexed by page-table row; the
 *      host page table is int32 [num_rows][ld]);
 *   3. plans the batch (rdx_plan_build with q_len 1 and written taken from
 *      row_written), uploads it, writes the new page-table entries to the
 *      device table and scatters k_new / v_new into the pools (one fused
 *      kernel), then runs decode attention into o (RDX_PLAN_DECODE plan);
 *   4. row_written[row[i]] = row_kv_len[row[i]].
 * node[i]: the locked node of request i (as in rdx_batch).  out_info (may be
 * NULL) receives the plan's sizes.  If io->dev_plan_bytes or
 * io->workspace_bytes is too small the call returns RDX_ENOBUFS with the
 * needed sizes in out_info, after returning the slots (the host arrays and
 * the free set are as before; leaves evicted to make room stay evicted):
 * grow the buffers and call again.  Other errors: EINVAL, ENOSPC, ESTATE,
 * EUNSUPPORTED, EDEVICE, with the same rollback.  Device work is enqueued on
 * `stream`; the call blocks only on the plan's staging ring (see
 * rdx_plan_upload). */
int rdx_decode_step(rdx_tree* tree, rdx_plan* plan, const rdx_attn_desc* desc, int32_t num_reqs,
                    const int64_t* node, const int32_t* row, int32_t* row_kv_len, int32_t* row_written,
                    int32_t* host_page_table, int64_t num_rows, int64_t ld, int32_t* out_slots,
                    const rdx_step_io* io, void* stream, rdx_plan_info* out_info);

/* A token-batched job run natively (BatchLLM explainer: Throughput-oriented
 * and Memory-centric Token Batching; Horizontal Fusion): the batcher of the
 * given groups (arguments as rdx_batcher_create) drives one attention launch
 * per iteration over `tree`.  Requests: 0..G-1 the groups' prefixes, G + m
 * member m; request r's full sequence is tokens[offsets[r] .. offsets[r+1])
 * (offsets[0] = 0): a prefix request holds its prefix, a member its prefix,
 * distinct prompt and generated tokens (decode_len of them).  The job keeps
 * its own host page table of num_rows x ld entries (row r of the device
 * page table mirrors row r).  The group arrays are copied; tokens and
 * offsets are borrowed and must stay valid until the job is destroyed.
 * flags:
 * RDX_JOB_KEEP_ROWS keeps every finished request's row (rdx_job_row);
 * RDX_JOB_DRY_RUN plans the iterations on the host only (no launch).
 * Per iteration:
 *   rdx_job_prepare -- the batcher's entries; admissions in entry order
 *     (match, lock, allocate the prompt's slots: a prefix request at its
 *     first chunk, a member at its first distinct chunk); one allocation for
 *     the decode tokens, in entry order; the plan of the batch (decode_plan
 *     when it holds decode tokens only, else extend_plan; query tokens in
 *     entry order, a chunk = positions begin .. begin+count-1 of its
 *     request).  *out_tokens = the batch's query tokens, 0 once the job is
 *     done; *out_kind = the plan kind; out_info (may be NULL) its sizes.
 *   rdx_job_launch -- io->q / k_new / v_new / o hold this iteration's
 *     tokens in entry order; one kernel stages the plan, writes the page
 *     table and scatters K/V, then the attention (+ merge).  RDX_ENOBUFS (no
 *     change, sizes in out_info) if io's plan or workspace buffer is small.
 *   rdx_job_complete -- the requests whose last token was in the batch are
 *     inserted (their full sequence, their row's slots), duplicates freed,
 *     unlocked, rows released; *out_finished = how many.
 * An error other than ENOBUFS leaves the job unusable (ESTATE afterwards):
 * destroy it (the tree keeps what was done). */
#define RDX_JOB_KEEP_ROWS 1
#define RDX_JOB_DRY_RUN 2
typedef struct rdx_job rdx_job;
int rdx_job_create(rdx_tree* tree, int32_t num_groups, const int32_t* prefix_len, const int32_t* member_offsets,
                   const int32_t* distinct_len, const int32_t* decode_len, int32_t s_chunk, int64_t m_threshold,
                   const int32_t* tokens, const int64_t* offsets, int32_t num_rows, int64_t ld, int32_t flags,
                   rdx_job** out);
void rdx_job_destroy(rdx_job* job);
int rdx_job_prepare(rdx_job* job, rdx_plan* extend_plan, rdx_plan* decode_plan, int64_t* out_tokens,
                    int32_t* out_kind, rdx_plan_info* out_info);
int rdx_job_complete(rdx_job* job, int32_t* out_finished);
/* A finished request's row (RDX_JOB_KEEP_ROWS): its length, the slots
 * (capacity cap; ENOBUFS with *out_len if short) and its matched length. */
int rdx_job_row(const rdx_job* job, int32_t req, int32_t* out, int64_t cap, int64_t* out_len, int64_t* out_matched);

/* The device part of one job iteration (see rdx_job_prepare). */
int rdx_job_launch(rdx_job* job, const rdx_attn_desc* desc, const rdx_step_io* io, void* stream,
                   rdx_plan_info* out_info);

/* ------------------------------------------------------- launch timing */
/* For benchmarks.  rdx_timing_begin(cap) starts recording: the next (up to
 * cap) attention launches are issued with HIP events bound to each kernel
 * dispatch itself (hipExtLaunchKernel) -- one pair on the attention kernel,
 * one on the merge kernel when the plan has split tiles -- so time the GPU
 * spends between dispatches is not counted.  rdx_timing_read waits for the
 * recorded launches and writes, in launch order (capacity cap), each
 * attention kernel's duration in milliseconds to out_attn_ms, the merge
 * kernel's (0 when none ran) to out_merge_ms (may be NULL) and the kind
 * (RDX_PLAN_EXTEND / RDX_PLAN_DECODE) to out_kind; it sets *out_n and stops
 * recording.  The recording is process-wide (launches from every thread and
 * plan count); one recording at a time.  rdx_timing_begin creates the
 * events for all cap launches itself (events persist for the process), so
 * the recorded launches create none: a caller that calls it once, and reads
 * with rdx_timing_read, before a timed region keeps event creation out of
 * that region.  Errors: EINVAL, EDEVICE. */
int rdx_timing_begin(int32_t cap);
int rdx_timing_read(float* out_attn_ms, float* out_merge_ms, int32_t* out_kind, int32_t cap,
                    int32_t* out_n);

#ifdef __cplusplus
}
#endif
#endif /* RDX_H */
