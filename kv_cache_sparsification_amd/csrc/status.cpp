// Error reporting of the C ABI: one message per calling thread.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "kvs_common.h"

namespace {
thread_local std::string g_last_error;
}

namespace kvs {

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVS_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return KVS_OK;
}

}  // namespace kvs

extern "C" const char* kvs_last_error(void) { return g_last_error.c_str(); }
extern "C" const char* kvs_version(void) { return "libkvs 0.1 (gfx950)"; }
