// Version and status strings of the C ABI declared in include/moe_ffn.h.
#include "common.h"

extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range";
    case MOE_ERR_ALIGN: return "a size is not a multiple of what the layout requires";
    case MOE_ERR_CAPACITY: return "M_cap cannot hold the worst-case grouped layout";
    case MOE_ERR_UNSUPPORTED: return "unsupported enum or parameter value";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_SCRATCH: return "the sizes need more than the entry point's static scratch";
    case MOE_ERR_DEVICE: return "the current device or its static scratch could not be queried";
    default: return "unknown status";
  }
}
