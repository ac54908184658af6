// Host-only stand-ins for the device entry points, linked ONLY into the
// sanitizer build of the host library (librdx_host_san.so), which has no
// HIP code.  Every device entry point fails with RDX_EUNSUPPORTED, so a test
// that reaches one under that build fails loudly instead of computing
// anything; rdx_plan_destroy releases a plan that was never uploaded.
#include "common.h"
#include "plan.h"
#include "rdx.h"

using namespace rdx;

namespace {
int no_device(const char* what) { return fail(RDX_EUNSUPPORTED, "%s: host-only sanitizer build has no device code", what); }
}  // namespace

extern "C" {

int rdx_kv_store(const rdx_attn_desc*, void*, void*, const void*, const void*, const int32_t*, int64_t, void*) {
  return no_device("rdx_kv_store");
}

int rdx_plan_upload(rdx_plan*, void*, int64_t, int32_t*, int64_t, void*) { return no_device("rdx_plan_upload"); }

void rdx_plan_destroy(rdx_plan* plan) { delete reinterpret_cast<Plan*>(plan); }

int rdx_extend_attention(const rdx_attn_desc*, const rdx_plan*, const void*, const void*, const void*, const void*,
                         const int32_t*, void*, void*, int64_t, void*) {
  return no_device("rdx_extend_attention");
}

int rdx_decode_attention(const rdx_attn_desc*, const rdx_plan*, const void*, const void*, const void*, const void*,
                         const int32_t*, void*, void*, int64_t, void*) {
  return no_device("rdx_decode_attention");
}

int rdx_decode_attention_noalloc(const rdx_attn_desc*, const rdx_plan*, const void*, const void*, const void*,
                                 const void*, const int32_t*, void*, void*) {
  return no_device("rdx_decode_attention_noalloc");
}

int rdx_decode_step(rdx_tree*, rdx_plan*, const rdx_attn_desc*, int32_t, const int64_t*, const int32_t*, int32_t*,
                    int32_t*, int32_t*, int64_t, int64_t, int32_t*, const rdx_step_io*, void*, rdx_plan_info*) {
  return no_device("rdx_decode_step");
}

int rdx_job_launch(rdx_job*, const rdx_attn_desc*, const rdx_step_io*, void*, rdx_plan_info*) {
  return no_device("rdx_job_launch");
}

// the timing calls check their arguments first, as the device build does
int rdx_timing_begin(int32_t cap) {
  if (cap < 0) return fail(RDX_EINVAL, "rdx_timing_begin: negative capacity");
  return no_device("rdx_timing_begin");
}

int rdx_timing_read(float* out_attn_ms, float*, int32_t* out_kind, int32_t cap, int32_t* out_n) {
  if (!out_n || cap < 0 || (cap > 0 && (!out_attn_ms || !out_kind)))
    return fail(RDX_EINVAL, "rdx_timing_read: bad arguments");
  return no_device("rdx_timing_read");
}

}  // extern "C"
