// Status codes, error text and the shared host-side argument checks.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace moev {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

bool need_ptr(const void* p, const char* name, unsigned align) {
  if (p == nullptr) {
    set_error("%s must not be NULL", name);
    return false;
  }
  return opt_ptr(p, name, align);
}

bool opt_ptr(const void* p, const char* name, unsigned align) {
  if (p != nullptr && (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0) {
    set_error("%s must be %u-byte aligned", name, align);
    return false;
  }
  return true;
}

bool check_dtype(int dt) {
  if (dt != MOEV_F32 && dt != MOEV_BF16) {
    set_error("unknown dtype %d", dt);
    return false;
  }
  return true;
}

moev_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return MOEV_ERR_HIP;
  }
  return MOEV_OK;
}

}  // namespace moev

extern "C" const char* moev_status_string(int status) {
  switch (status) {
    case MOEV_OK: return "ok";
    case MOEV_ERR_INVALID_ARG: return "invalid argument";
    case MOEV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOEV_ERR_WORKSPACE: return "workspace missing or too small";
    case MOEV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" const char* moev_last_error(void) { return moev::g_last_error.c_str(); }

extern "C" int moev_version(void) { return 100; }  // 0.1.0
