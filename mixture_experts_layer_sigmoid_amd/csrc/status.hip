// Status codes, per-thread error messages and ABI version.
#include "common.h"

#include <cstdio>

namespace moe {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    char buf[256];
    snprintf(buf, sizeof(buf), "%s: %s", what, hipGetErrorString(e));
    return fail(MOE_ERR_HIP, buf);
  }
  return MOE_OK;
}

}  // namespace moe

extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

extern "C" const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported format combination";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer or row size";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" const char* moe_last_error(void) { return moe::g_last_error.c_str(); }
