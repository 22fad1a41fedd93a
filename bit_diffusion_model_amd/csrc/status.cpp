// Error reporting and shared argument checks of the C ABI (host code only: built by the
// host compiler, so the host pack can also be built alone, e.g. under sanitizers).
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/svdq.h"
#include "internal.hpp"

namespace svdq {

static thread_local std::string g_err;

svdq_status fail(svdq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

svdq_status ok() {
  g_err.clear();
  return SVDQ_OK;
}

int group_of(int fmt) { return fmt == SVDQ_INT4_G64 ? 64 : (fmt == SVDQ_NVFP4_G16 ? 16 : 32); }

svdq_status check_dims(int64_t K, int64_t N, int32_t fmt) {
  if (fmt != SVDQ_INT4_G64 && fmt != SVDQ_MXFP4_G32 && fmt != SVDQ_NVFP4_G16)
    return fail(SVDQ_EUNSUPPORTED, "unsupported format %d", (int)fmt);
  if (K < 128 || K % 128 != 0) return fail(SVDQ_EINVAL, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (N < 1) return fail(SVDQ_EINVAL, "N must be >= 1 (got %lld)", (long long)N);
  return SVDQ_OK;
}

}  // namespace svdq

extern "C" const char* svdq_last_error(void) { return svdq::g_err.c_str(); }
