// Host side of the device entry points of librdx: argument checks, plan
// upload (pinned staging, page-table writes), the attention launches and
// launch timing.  The kernels are in attn_kernels.h.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "attn_kernels.h"
#include "common.h"
#include "job.h"
#include "plan.h"
#include "radix_tree.h"


using namespace rdx;

// Device-resident workspace of rdx_decode_attention_noalloc: the partial
// (o, max, sum) states of split tiles.  One copy per GPU, held until the
// process ends.  Host code never passes this name to a kernel (in host code
// it is a stand-in, not a device address): it uses the per-device address
// from hipGetSymbolAddress instead.
constexpr int64_t kNoAllocScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of `scratch` on the current device, looked up once per device
// with that device current (the first call on the device).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RDX_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(RDX_EUNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(RDX_EDEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

// Launch timing state (see rdx_timing_begin): per launch one event pair
// bound to the attention dispatch and, for plans with split tiles, one bound
// to the merge dispatch; events are reused across runs.
struct Timing {
  bool on = false;
  int32_t cap = 0;
  std::vector<hipEvent_t> ev;  // 4 per launch: attention start/stop, merge start/stop
  std::vector<int32_t> kind, has_merge;
  int32_t used = 0;
} g_timing;

// Adds one launch's four events to the recording state.  On a failed
// creation the events made so far are destroyed and nothing is added, so
// the state keeps four events per launch slot.
hipError_t add_timing_slot() {
  hipEvent_t x[4];
  for (int k = 0; k < 4; ++k) {
    hipError_t e = hipEventCreate(&x[k]);
    if (e != hipSuccess) {
      for (int j = 0; j < k; ++j) (void)hipEventDestroy(x[j]);
      return e;
    }
  }
  g_timing.ev.insert(g_timing.ev.end(), x, x + 4);
  g_timing.kind.push_back(0);
  g_timing.has_merge.push_back(0);
  return hipSuccess;
}

// Launches the attention kernel and, for plans with split tiles, the merge
// kernel behind it; while timing is on, each dispatch carries its own events.
// untimed: never record (the no-allocation entry point creates no events)
template <typename KA, typename KM>
hipError_t launch(KA attn, KM merge, int64_t n_items, int64_t n_merge, hipStream_t st, int32_t kind,
                  const AttnArgs& a, int threads = kThreads, bool untimed = false) {
  hipEvent_t* ev = nullptr;
  if (!untimed && g_timing.on && g_timing.used < g_timing.cap) {
    const int32_t i = g_timing.used;
    while ((int32_t)g_timing.kind.size() <= i) {
      hipError_t e = add_timing_slot();
      if (e != hipSuccess) return e;
    }
    g_timing.kind[i] = kind;
    g_timing.has_merge[i] = n_merge > 0;
    g_timing.used++;
    ev = &g_timing.ev[4 * (size_t)i];
  }
  const dim3 block(kThreads), ablock(threads);
  if (ev)
    hipExtLaunchKernelGGL(attn, dim3((unsigned)n_items), ablock, 0, st, ev[0], ev[1], 0, a);
  else
    hipLaunchKernelGGL(attn, dim3((unsigned)n_items), ablock, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_merge == 0) return e;
  if (ev)
    hipExtLaunchKernelGGL(merge, dim3((unsigned)n_merge), block, 0, st, ev[2], ev[3], 0, a);
  else
    hipLaunchKernelGGL(merge, dim3((unsigned)n_merge), block, 0, st, a);
  return hipGetLastError();
}

int hip_fail(hipError_t e, const char* what) { return fail(RDX_EDEVICE, "%s: %s", what, hipGetErrorString(e)); }

bool same_shape(const rdx_attn_desc& a, const rdx_attn_desc& b) {
  return a.dtype == b.dtype && a.num_q_heads == b.num_q_heads && a.num_kv_heads == b.num_kv_heads &&
         a.head_dim == b.head_dim && a.num_slots == b.num_slots;
}

int launch_attention(const rdx_attn_desc* desc, const rdx_plan* hplan, int32_t kind, const void* dev_plan,
                     const void* q, const void* kp, const void* vp, const int32_t* pt, void* o, void* ws,
                     int64_t ws_bytes, void* stream, bool untimed = false) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!hplan) return fail(RDX_EINVAL, "attention: null plan");
  const Plan* p = reinterpret_cast<const Plan*>(hplan);
  if (!p->built) return fail(RDX_ESTATE, "attention: plan not built");
  if (p->kind != kind) return fail(RDX_EINVAL, "attention: plan kind %d does not match this entry point", p->kind);
  if (!same_shape(*desc, p->desc)) return fail(RDX_EINVAL, "attention: descriptor differs from the plan's");
  // workgroups: every item record once per KV head
  const int64_t n_items = (int64_t)p->items.size() / kItemWords * desc->num_kv_heads;
  if (n_items == 0) return ok();
  if (!dev_plan || !q || !kp || !vp || !pt || !o) return fail(RDX_EINVAL, "attention: null device pointer");
  if (p->ws_bytes > 0 && (!ws || ws_bytes < p->ws_bytes))
    return fail(RDX_EINVAL, "attention: workspace of %lld bytes needed", (long long)p->ws_bytes);
  const int64_t n_merge = (int64_t)(p->mblocks.size() / kMBlockWords) * desc->num_kv_heads;
  if (p->ws_tokens * desc->num_q_heads >= ((int64_t)1 << 31))
    return fail(RDX_EUNSUPPORTED, "attention: split workspace too large (%lld partial rows)",
                (long long)(p->ws_tokens * desc->num_q_heads));
  if (n_items > INT32_MAX || n_merge > INT32_MAX) return fail(RDX_EINVAL, "attention: too many work items");
  const int32_t* base = reinterpret_cast<const int32_t*>(dev_plan);
  AttnArgs a;
  a.items = base + p->off_items;
  a.tiles = base + p->off_tiles;
  a.jobs = base + p->off_jobs;
  a.toks = base + p->off_toks;
  a.contribs = base + p->off_contribs;
  a.cptr = base + p->off_cptr;
  a.clist = base + p->off_clist;
  a.mblocks = base + p->off_mblocks;
  a.page_table = pt;
  a.ld = p->ld;
  a.q = q;
  a.kp = kp;
  a.vp = vp;
  a.o = o;
  char* wsb = reinterpret_cast<char*>(ws);
  a.ws_o = reinterpret_cast<float*>(wsb);
  a.ws_ml = wsb ? reinterpret_cast<float*>(wsb + p->ws_ml_offset) : nullptr;
  a.ws_tokens = p->ws_tokens;
  a.row_bytes = (int32_t)(kv_row_elems(desc) * kv_elem_bytes(desc));
  a.pool_bytes = desc->num_slots * a.row_bytes;
  a.hq = desc->num_q_heads;
  a.hkv = desc->num_kv_heads;
  a.group = a.hq / a.hkv;
  const float scale = desc->sm_scale > 0.f ? desc->sm_scale : 1.f / sqrtf((float)desc->head_dim);
  a.scale_log2 = scale * kLog2e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  // pools under 2 GiB are addressed with 32-bit buffer offsets (the buffer
  // resource's record count is a signed 32-bit value here)
  const bool off32 = a.pool_bytes < ((int64_t)1 << 31);
  if (desc->dtype == RDX_BF16 && p->tile_rows == kDecodeTileRows) {
    if (desc->head_dim == 128)
      e = off32 ? launch(attn_decode_kernel<128, true>, merge_kernel<__bf16, 128>, n_items, n_merge, st, kind, a, kThreads, untimed)
                : launch(attn_decode_kernel<128, false>, merge_kernel<__bf16, 128>, n_items, n_merge, st, kind, a, kThreads, untimed);
    else
      e = off32 ? launch(attn_decode_kernel<64, true>, merge_kernel<__bf16, 64>, n_items, n_merge, st, kind, a, kThreads, untimed)
                : launch(attn_decode_kernel<64, false>, merge_kernel<__bf16, 64>, n_items, n_merge, st, kind, a, kThreads, untimed);
  } else if (desc->dtype == RDX_BF16 && p->tile_rows == 256) {
    e = off32 ? launch(attn_bf16_wide_kernel<true>, merge_kernel<__bf16, 128>, n_items, n_merge, st, kind, a,
                       kWideThreads, untimed)
              : launch(attn_bf16_wide_kernel<false>, merge_kernel<__bf16, 128>, n_items, n_merge, st, kind, a,
                       kWideThreads, untimed);
  } else if (desc->dtype == RDX_BF16) {
    if (desc->head_dim == 128)
      e = off32 ? launch(attn_bf16_kernel<128, true>, merge_kernel<__bf16, 128>, n_items, n_merge, st, kind, a, kThreads, untimed)
                : launch(attn_bf16_kernel<128, false>, merge_kernel<__bf16, 128>, n_items, n_merge, st, kind, a, kThreads, untimed);
    else
      e = off32 ? launch(attn_bf16_kernel<64, true>, merge_kernel<__bf16, 64>, n_items, n_merge, st, kind, a, kThreads, untimed)
                : launch(attn_bf16_kernel<64, false>, merge_kernel<__bf16, 64>, n_items, n_merge, st, kind, a, kThreads, untimed);
  }
  else
    e = desc->head_dim == 128 ? launch(attn_f32_kernel<128>, merge_kernel<float, 128>, n_items, n_merge, st, kind, a, kThreads, untimed)
                              : launch(attn_f32_kernel<64>, merge_kernel<float, 64>, n_items, n_merge, st, kind, a, kThreads, untimed);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

// Marks the current staging buffer in use until the work queued so far on
// `st` (the copy or kernel that reads it) has completed.
int stage_done(Plan* p, hipStream_t st) {
  Plan::Stage& sg = p->stages[p->uploads % p->n_stages];
  hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(sg.event), st);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  sg.pending = true;
  p->uploads++;
  return ok();
}

// Plan upload: checks, staging through the plan's pinned ring, the copy to
// the device (a kernel reading the mapped staging buffer) and (write_pt) the
// page-table write kernel.
// zero_copy: stage only (no copy, no page-table kernel, no event): the
// caller launches a kernel that reads the staging buffer through
// *out_stage_dev and then calls stage_done() behind it.
int upload_plan(Plan* p, void* dev_plan, int64_t dev_plan_bytes, int32_t* page_table, int64_t page_table_rows,
                hipStream_t st, bool write_pt, bool zero_copy = false, const int32_t** out_stage_dev = nullptr) {
  if (!p->built) return fail(RDX_ESTATE, "rdx_plan_upload: plan not built");
  const int64_t bytes = p->total_words * 4;
  if (dev_plan_bytes < bytes) return fail(RDX_EINVAL, "rdx_plan_upload: device buffer of %lld bytes needed", (long long)bytes);
  const int64_t n_runs = (int64_t)p->runs.size() / kRunWords;
  if (n_runs > 0 && (!page_table || page_table_rows <= p->max_page_row))
    return fail(RDX_EINVAL, "rdx_plan_upload: page table with more than %lld rows needed", (long long)p->max_page_row);
  hipError_t e;
  Plan::Stage& sg = p->stages[p->uploads % p->n_stages];
  if (!sg.event) {
    hipEvent_t ev;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    sg.event = ev;
  }
  if (sg.pending) {
    e = hipEventSynchronize(reinterpret_cast<hipEvent_t>(sg.event));
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    sg.pending = false;
  }
  if (sg.bytes < bytes) {
    // every stage of the ring grows at once (pinning memory is slow: one
    // stall per new size, not one per stage), and outgrown buffers are freed
    // with the plan (freeing pinned memory waits for the device; a buffer
    // still read by a queued copy stays valid)
    const int64_t want = bytes + bytes / 2 + 4096;
    for (int i = 0; i < p->n_stages; ++i) {
      Plan::Stage& o = p->stages[i];
      if (o.bytes >= want) continue;
      if (o.pinned) p->retired.push_back(o.pinned);
      o.pinned = nullptr;
      o.bytes = 0;
      e = hipHostMalloc(&o.pinned, want, hipHostMallocDefault);
      if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
      o.bytes = want;
      e = hipHostGetDevicePointer(&o.pinned_dev, o.pinned, 0);
      if (e != hipSuccess) return hip_fail(e, "hipHostGetDevicePointer");
    }
  }
  int32_t* h = reinterpret_cast<int32_t*>(sg.pinned);
  auto put = [&](int64_t off, const std::vector<int32_t>& v) {
    if (!v.empty()) memcpy(h + off, v.data(), v.size() * 4);
  };
  put(p->off_items, p->items);
  put(p->off_tiles, p->tiles);
  put(p->off_jobs, p->jobs);
  put(p->off_toks, p->toks);
  put(p->off_contribs, p->contribs);
  put(p->off_runs, p->runs);
  put(p->off_run_slots, p->run_slots);
  put(p->off_new, p->new_slots);
  put(p->off_cptr, p->cptr);
  put(p->off_clist, p->clist);
  put(p->off_mblocks, p->mblocks);
  if (zero_copy) {
    *out_stage_dev = reinterpret_cast<const int32_t*>(sg.pinned_dev);
    return ok();
  }
  const int64_t n_vec4 = (p->total_words + 3) / 4;  // total_words is a multiple of 16
  int64_t n_copy = (n_vec4 + 255) / 256;
  if (n_copy > 512) n_copy = 512;
  hipLaunchKernelGGL(plan_copy_kernel, dim3((unsigned)n_copy), dim3(256), 0, st,
                     reinterpret_cast<const int4*>(sg.pinned_dev), reinterpret_cast<int4*>(dev_plan), n_vec4);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "plan copy launch");
  if (write_pt && n_runs > 0) {
    const int32_t* db = reinterpret_cast<const int32_t*>(dev_plan);
    hipLaunchKernelGGL(page_table_write_kernel, dim3((unsigned)n_runs), dim3(256), 0, st, page_table, p->ld,
                       db + p->off_runs, db + p->off_run_slots);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "page-table write launch");
  }
  return stage_done(p, st);
}

}  // namespace

extern "C" {

int rdx_kv_store(const rdx_attn_desc* desc, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                 const int32_t* slots, int64_t n, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (n < 0) return fail(RDX_EINVAL, "rdx_kv_store: negative n");
  if (n == 0) return ok();
  if (!k_pool || !v_pool || !k_new || !v_new || !slots) return fail(RDX_EINVAL, "rdx_kv_store: null pointer");
  const int64_t esize = desc->dtype == RDX_BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)desc->num_kv_heads * desc->head_dim * esize;
  if (row_bytes % 16) return fail(RDX_EUNSUPPORTED, "rdx_kv_store: row of %lld bytes", (long long)row_bytes);
  const int64_t row_vecs = row_bytes / 16;
  const int64_t total = n * row_vecs;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<uint4*>(k_pool), reinterpret_cast<uint4*>(v_pool),
                     reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new), slots, n, row_vecs,
                     kv_row_elems(desc) * esize / 16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "rdx_kv_store launch");
  return ok();
}

int rdx_plan_upload(rdx_plan* hplan, void* dev_plan, int64_t dev_plan_bytes, int32_t* page_table,
                    int64_t page_table_rows, void* stream) {
  if (!hplan || !dev_plan) return fail(RDX_EINVAL, "rdx_plan_upload: null argument");
  return upload_plan(reinterpret_cast<Plan*>(hplan), dev_plan, dev_plan_bytes, page_table, page_table_rows,
                     reinterpret_cast<hipStream_t>(stream), true);
}

void rdx_plan_destroy(rdx_plan* hplan) {
  if (!hplan) return;
  Plan* p = reinterpret_cast<Plan*>(hplan);
  // teardown has no caller to report to: each buffer is released whatever
  // the status of the calls before it (a copy still reading a staging
  // buffer is waited for first)
  for (Plan::Stage& sg : p->stages) {
    if (sg.pending && sg.event) (void)hipEventSynchronize(reinterpret_cast<hipEvent_t>(sg.event));
    if (sg.event) (void)hipEventDestroy(reinterpret_cast<hipEvent_t>(sg.event));
    if (sg.pinned) (void)hipHostFree(sg.pinned);
  }
  for (void* r : p->retired) (void)hipHostFree(r);
  delete p;
}

int rdx_extend_attention(const rdx_attn_desc* desc, const rdx_plan* plan, const void* dev_plan, const void* q,
                         const void* k_pool, const void* v_pool, const int32_t* page_table, void* o, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  return launch_attention(desc, plan, RDX_PLAN_EXTEND, dev_plan, q, k_pool, v_pool, page_table, o, workspace,
                          workspace_bytes, stream);
}

int rdx_decode_attention(const rdx_attn_desc* desc, const rdx_plan* plan, const void* dev_plan, const void* q,
                         const void* k_pool, const void* v_pool, const int32_t* page_table, void* o, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  return launch_attention(desc, plan, RDX_PLAN_DECODE, dev_plan, q, k_pool, v_pool, page_table, o, workspace,
                          workspace_bytes, stream);
}

int rdx_decode_attention_noalloc(const rdx_attn_desc* desc, const rdx_plan* plan, const void* dev_plan,
                                 const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                                 void* o, void* stream) {
  if (!plan) return fail(RDX_EINVAL, "rdx_decode_attention_noalloc: null plan");
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  if (p->ws_bytes > kNoAllocScratchBytes)
    return fail(RDX_EINVAL, "rdx_decode_attention_noalloc: the plan's split tiles need %lld bytes of workspace, "
                "the built-in workspace holds %lld", (long long)p->ws_bytes, (long long)kNoAllocScratchBytes);
  void* ws = nullptr;
  if (p->ws_bytes > 0) {
    int rc = scratch_address(&ws);
    if (rc) return rc;
  }
  return launch_attention(desc, plan, RDX_PLAN_DECODE, dev_plan, q, k_pool, v_pool, page_table, o, ws,
                          p->ws_bytes > 0 ? kNoAllocScratchBytes : 0, stream, /*untimed=*/true);
}

// The device tail of a step whose plan is built: the work list staged in
// mapped pinned memory, ONE kernel that copies it to the device plan buffer,
// writes the page-table entries and scatters the num_new new K/V rows into
// their slots, then the attention (+ merge) launch of `kind`.
static int store_and_attend(Plan* p, rdx_plan* hplan, const rdx_attn_desc* desc, int32_t kind, const rdx_step_io* io,
                            void* stream, int64_t ld, int64_t num_new) {
  const int64_t esize = desc->dtype == RDX_BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)desc->num_kv_heads * desc->head_dim * esize;
  if (row_bytes % 16) return fail(RDX_EUNSUPPORTED, "step: KV row of %lld bytes", (long long)row_bytes);
  if (!io->dev_plan || !io->page_table || !io->k_pool || !io->v_pool || !io->q || !io->k_new || !io->v_new || !io->o)
    return fail(RDX_EINVAL, "step: null device pointer");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t n_runs = (int64_t)p->runs.size() / kRunWords;
  const int64_t row_vecs = row_bytes / 16, total = num_new * row_vecs;
  const int64_t pitch_vecs = kv_row_elems(desc) * esize / 16;
  // The fused kernel reads the staged list through PCIe: right for a decode
  // step (a few KB, one page-table entry per run).  A batch that admits
  // requests writes whole rows and carries a large list: copy it by DMA,
  // then write the page table and scatter K/V from device memory.
  if ((int64_t)p->run_slots.size() > n_runs + 256 || p->total_words > (int64_t)1 << 18) {
    int rc = upload_plan(p, io->dev_plan, io->dev_plan_bytes, io->page_table, io->page_table_rows, st, true);
    if (rc) return rc;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (total > 0) {
      hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)blocks), dim3(256), 0, st, reinterpret_cast<uint4*>(io->k_pool),
                         reinterpret_cast<uint4*>(io->v_pool), reinterpret_cast<const uint4*>(io->k_new),
                         reinterpret_cast<const uint4*>(io->v_new),
                         reinterpret_cast<const int32_t*>(io->dev_plan) + p->off_new, num_new, row_vecs, pitch_vecs);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "KV store launch");
    }
    return launch_attention(desc, hplan, kind, io->dev_plan, io->q, io->k_pool, io->v_pool, io->page_table, io->o,
                            io->workspace, io->workspace_bytes, stream);
  }
  const int32_t* hs = nullptr;  // the staged work list, device-addressable
  int rc = upload_plan(p, io->dev_plan, io->dev_plan_bytes, io->page_table, io->page_table_rows, st, false, true, &hs);
  if (rc) return rc;
  const int64_t n_vec4 = (p->total_words + 3) / 4;  // total_words is a multiple of 16
  int64_t n_copy = (n_vec4 + 255) / 256;
  if (n_copy > 64) n_copy = 64;
  int64_t kv_blocks = (total + 255) / 256;
  if (kv_blocks > 65536) kv_blocks = 65536;
  const int64_t n_pt = (n_runs + 255) / 256;
  hipLaunchKernelGGL(step_store_kernel, dim3((unsigned)(n_copy + n_pt + kv_blocks)), dim3(256), 0, st,
                     reinterpret_cast<const int4*>(hs), reinterpret_cast<int4*>(io->dev_plan), n_vec4,
                     (int32_t)n_copy, io->page_table, ld, hs + p->off_runs, hs + p->off_run_slots, (int32_t)n_runs,
                     reinterpret_cast<uint4*>(io->k_pool), reinterpret_cast<uint4*>(io->v_pool),
                     reinterpret_cast<const uint4*>(io->k_new), reinterpret_cast<const uint4*>(io->v_new),
                     hs + p->off_new, num_new, row_vecs, pitch_vecs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "step store launch");
  rc = stage_done(p, st);
  if (rc) return rc;
  return launch_attention(desc, hplan, kind, io->dev_plan, io->q, io->k_pool, io->v_pool, io->page_table, io->o,
                          io->workspace, io->workspace_bytes, stream);
}

int rdx_job_launch(rdx_job* j, const rdx_attn_desc* desc, const rdx_step_io* io, void* stream,
                   rdx_plan_info* out_info) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!j || !io) return fail(RDX_EINVAL, "rdx_job_launch: bad arguments");
  if (j->broken) return fail(RDX_ESTATE, "rdx_job_launch: an earlier error left the job inconsistent");
  if (j->state != 1) return fail(RDX_ESTATE, "rdx_job_launch: no prepared iteration");
  if (j->dry_run) return fail(RDX_ESTATE, "rdx_job_launch: a dry-run job launches nothing");
  Plan* p = j->plan;
  if (!same_shape(*desc, p->desc)) return fail(RDX_EINVAL, "rdx_job_launch: descriptor differs from the plan's");
  rdx_plan_info info;
  p->fill_info(&info);
  if (out_info) *out_info = info;
  if (io->dev_plan_bytes < info.device_bytes || (info.workspace_bytes > 0 && io->workspace_bytes < info.workspace_bytes))
    return fail(RDX_ENOBUFS, "rdx_job_launch: buffers of %lld (plan) and %lld (workspace) bytes needed",
                (long long)info.device_bytes, (long long)info.workspace_bytes);
  if (io->page_table_rows < j->num_rows)
    return fail(RDX_EINVAL, "rdx_job_launch: device page table has %lld rows, the job uses %d",
                (long long)io->page_table_rows, j->num_rows);
  rc = store_and_attend(p, reinterpret_cast<rdx_plan*>(p), desc, j->kind, io, stream, j->ld, j->n_tokens);
  if (rc) {
    j->broken = true;
    return rc;
  }
  j->state = 2;
  return ok();
}

int rdx_decode_step(rdx_tree* tree, rdx_plan* hplan, const rdx_attn_desc* desc, int32_t num_reqs,
                    const int64_t* node, const int32_t* row, int32_t* row_kv_len, int32_t* row_written,
                    int32_t* host_page_table, int64_t num_rows, int64_t ld, int32_t* out_slots,
                    const rdx_step_io* io, void* stream, rdx_plan_info* out_info) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!tree || !hplan || !io || num_reqs < 0 || num_rows <= 0 || ld <= 0)
    return fail(RDX_EINVAL, "rdx_decode_step: bad arguments");
  if (num_reqs > 0 && (!node || !row || !row_kv_len || !row_written || !host_page_table || !out_slots))
    return fail(RDX_EINVAL, "rdx_decode_step: null array");
  Plan* p = reinterpret_cast<Plan*>(hplan);
  if (p->kind != RDX_PLAN_DECODE) return fail(RDX_EINVAL, "rdx_decode_step: not a decode plan");
  if (!same_shape(*desc, p->desc)) return fail(RDX_EINVAL, "rdx_decode_step: descriptor differs from the plan's");
  // per-request lengths in batch order (thread-local scratch: no allocation per step)
  thread_local std::vector<int32_t> kv, wr, ql;
  kv.resize(num_reqs);
  wr.resize(num_reqs);
  ql.assign(num_reqs, 1);
  for (int32_t i = 0; i < num_reqs; ++i) {
    const int32_t r = row[i];
    if (r < 0 || r >= num_rows) return fail(RDX_EINVAL, "rdx_decode_step: request %d: row %d out of range", i, r);
    if (row_kv_len[r] < 0 || row_kv_len[r] >= ld)
      return fail(RDX_EINVAL, "rdx_decode_step: request %d: row %d is full", i, r);
    kv[i] = row_kv_len[r] + 1;
    wr[i] = row_written[r];
  }
  RadixTree& t = tree->impl;
  rc = t.alloc(num_reqs, out_slots);
  if (rc) return rc;
  auto undo = [&](int code) {
    // hand the slots back (the free set is as before the call); the error
    // message of `code` is kept
    std::string msg = last_error();
    t.free_slots(out_slots, num_reqs);
    last_error() = msg;
    return code;
  };
  rdx_batch b{num_reqs, 0, node, row, kv.data(), ql.data(), wr.data(), out_slots};
  p->ld = ld;
  rc = p->build(t, b, ld);
  if (rc) return undo(rc);
  rdx_plan_info info;
  p->fill_info(&info);
  if (out_info) *out_info = info;
  if (io->dev_plan_bytes < info.device_bytes || (info.workspace_bytes > 0 && io->workspace_bytes < info.workspace_bytes))
    return undo(fail(RDX_ENOBUFS, "rdx_decode_step: buffers of %lld (plan) and %lld (workspace) bytes needed",
                     (long long)info.device_bytes, (long long)info.workspace_bytes));
  if (num_reqs > 0 && (!io->dev_plan || !io->page_table || !io->k_pool || !io->v_pool || !io->q || !io->k_new ||
                       !io->v_new || !io->o))
    return undo(fail(RDX_EINVAL, "rdx_decode_step: null device pointer"));
  if (num_reqs > 0) {
    rc = store_and_attend(p, hplan, desc, RDX_PLAN_DECODE, io, stream, ld, num_reqs);
    if (rc) return undo(rc);
  }
  // commit: the new slots into the host page-table rows, lengths, written counts
  for (int32_t i = 0; i < num_reqs; ++i) {
    const int32_t r = row[i];
    host_page_table[(int64_t)r * ld + row_kv_len[r]] = out_slots[i];
    row_kv_len[r] = kv[i];
    row_written[r] = kv[i];
  }
  return ok();
}

int rdx_timing_begin(int32_t cap) {
  if (cap < 0) return fail(RDX_EINVAL, "rdx_timing_begin: negative capacity");
  // every event the recording can need is created here, so the launches it
  // records create none (event creation costs the host microseconds per
  // event, which a host-paced launch sequence would otherwise absorb)
  while ((int32_t)g_timing.kind.size() < cap) {
    hipError_t e = add_timing_slot();
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  g_timing.on = true;
  g_timing.cap = cap;
  g_timing.used = 0;
  return ok();
}

int rdx_timing_read(float* out_attn_ms, float* out_merge_ms, int32_t* out_kind, int32_t cap, int32_t* out_n) {
  if (!out_n || cap < 0 || (cap > 0 && (!out_attn_ms || !out_kind)))
    return fail(RDX_EINVAL, "rdx_timing_read: bad arguments");
  const int32_t n = g_timing.used < cap ? g_timing.used : cap;
  for (int32_t i = 0; i < n; ++i) {
    const hipEvent_t* ev = &g_timing.ev[4 * (size_t)i];
    const bool m = g_timing.has_merge[i] != 0;
    hipError_t e = hipEventSynchronize(m ? ev[3] : ev[1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    e = hipEventElapsedTime(&out_attn_ms[i], ev[0], ev[1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    if (out_merge_ms) {
      out_merge_ms[i] = 0.f;
      if (m) {
        e = hipEventElapsedTime(&out_merge_ms[i], ev[2], ev[3]);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      }
    }
    out_kind[i] = g_timing.kind[i];
  }
  *out_n = n;
  g_timing.on = false;
  g_timing.used = 0;
  return ok();
}

}  // extern "C"
