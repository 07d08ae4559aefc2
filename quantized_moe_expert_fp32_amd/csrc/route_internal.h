// Routing launchers shared with the fused decode-layer entry point.
#pragma once

#include "moe_internal.h"

namespace moe {

moe_status check_route_outputs(const moe_shape& sh, int T, const int32_t* ids, const uint16_t* w,
                               const uint16_t* wsh);

// Router logits and selection in one launch for T <= 16 (the last workgroup to
// finish selects); `counter` is a zero-initialised device word left at zero.
moe_status launch_route_fused(const moe_shape& sh, const void* router_packed, const float* logit_bias,
                              const uint16_t* x, int T, float* logits, unsigned int* counter, int32_t* ids,
                              uint16_t* w, uint16_t* wsh, hipStream_t hs);

}  // namespace moe
