// Status strings and ABI version of libmoe.so.
#include "common.h"

MOE_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument (size, null or misaligned pointer, stride)";
    case MOE_ERR_DTYPE: return "unsupported dtype";
    case MOE_ERR_CAPACITY: return "buffer smaller than the static row bound";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    default: return "unknown status";
  }
}

MOE_API int moe_abi_version(void) { return 12; }
