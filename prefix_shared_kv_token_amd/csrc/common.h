// Shared host-side helpers of librdx: status codes and the thread-local
// error message returned by rdx_last_error().
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "rdx.h"

namespace rdx {

std::string& last_error();

inline int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error() = buf;
  return code;
}

inline int ok() {
  last_error().clear();
  return RDX_OK;
}

// Validates an attention descriptor (dtype, heads, head_dim, pool size, row pitch).
int check_desc(const rdx_attn_desc* d);

inline int64_t kv_elem_bytes(const rdx_attn_desc* d) { return d->dtype == RDX_BF16 ? 2 : 4; }
// Elements from one slot's row of a KV pool to the next.
inline int64_t kv_row_elems(const rdx_attn_desc* d) {
  return d->kv_row_pitch > 0 ? d->kv_row_pitch : (int64_t)d->num_kv_heads * d->head_dim;
}

}  // namespace rdx
