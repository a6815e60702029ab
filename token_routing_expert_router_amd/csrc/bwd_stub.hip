#include "common.h"
extern "C" size_t moe_expert_ffn_bwd_workspace_size(int32_t, int64_t, int64_t, int64_t, moe_dtype_t) { return 0; }
extern "C" moe_status_t moe_expert_ffn_bwd(const void *, const void *, const void *, const int32_t *, const void *, const void *, int32_t, int64_t, int64_t, int64_t, moe_dtype_t, void *, float *, float *, void *, size_t, void *) { return MOE_ERR_UNSUPPORTED; }
extern "C" size_t moe_route_bwd_workspace_size(int64_t, int64_t, int32_t, int32_t) { return 0; }
extern "C" moe_status_t moe_route_bwd(const void *, const int32_t *, const float *, const float *, int64_t, int64_t, int32_t, int32_t, moe_dtype_t, float *, float *, void *, size_t, void *) { return MOE_ERR_UNSUPPORTED; }
