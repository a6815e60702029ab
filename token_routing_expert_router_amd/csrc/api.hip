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

extern "C" size_t moe_workspace_size(moe_op_t op, int64_t T, int32_t E, int32_t k,
                                     const moe_layout_t *layout, int64_t rows, int64_t d,
                                     int64_t F, moe_dtype_t dtype) {
    switch (op) {
    case MOE_OP_DISPATCH: return moe_dispatch_workspace_size(T, E, k, layout);
    case MOE_OP_EXPERT_FFN: return moe_expert_ffn_workspace_size(E, rows, d, F, dtype);
    case MOE_OP_EXPERT_FFN_BWD: return moe_expert_ffn_bwd_workspace_size(E, rows, d, F, dtype);
    default: return 0;
    }
}
