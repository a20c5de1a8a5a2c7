// Thread-local error text behind wf_last_error(). Host only; builds with g++ or hipcc.
#include "wf_error.h"

#include <cstdio>

#include "wf_attn.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace wf {
int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}
void clear_error() { g_last_error[0] = '\0'; }
}  // namespace wf

extern "C" const char* wf_last_error(void) { return g_last_error; }
extern "C" int32_t wf_abi_version(void) { return WF_ABI_VERSION; }
