// Status strings and ABI version of libmoe.
#include "common.h"

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or mode";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

extern "C" int moe_abi_version(void) { return 6; }
