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

// Validates an attention descriptor (dtype, heads, head_dim, pool size).
int check_desc(const rdx_attn_desc* d);

}  // namespace rdx
