// Per-thread error message and version query of the C ABI.
#include "common.hpp"

#include <string.h>

namespace sdq {

static thread_local char g_err[512] = {0};

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: HIP error %d (%s)", what, int(e), hipGetErrorString(e));
    return SDQ_EHIP;
  }
  return SDQ_OK;
}

}  // namespace sdq

extern "C" const char* sdq_last_error(void) { return sdq::g_err; }

extern "C" int sdq_abi_version(void) { return 3; }
