#include "status.h"

#include <cstdio>
#include <string>

namespace pagedkv {
namespace {
thread_local std::string g_last_error;
}

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return PAGED_OK;
}

}  // namespace pagedkv

extern "C" int32_t paged_abi_version(void) { return PAGEDKV_ABI_VERSION; }

extern "C" const char* paged_last_error(void) { return pagedkv::g_last_error.c_str(); }
