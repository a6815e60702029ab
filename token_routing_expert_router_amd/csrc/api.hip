// Library-wide entry points: ABI version and status strings.
#include "common.h"

extern "C" int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

extern "C" const char *moe_status_str(moe_status_t s) {
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_SHAPE: return "inconsistent shapes";
    case MOE_ERR_ALIGN: return "row length or pointer not 16-byte aligned";
    case MOE_ERR_CAPACITY: return "workspace or destination region too small";
    case MOE_ERR_BAD_INDEX: return "expert id out of range or repeated within a token";
    case MOE_ERR_HIP: return "HIP launch or query failed";
    case MOE_ERR_UNSUPPORTED: return "sizes outside what the kernels implement";
    default: return "unknown status";
    }
}
