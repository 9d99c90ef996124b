// ABI-level helpers of libmoe: version and status names.
#include "moe_internal.h"

MOE_EXPORT int moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_EXPORT const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or alignment";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_DEVICE: return "HIP launch or device error";
    default: return "unknown status";
  }
}
