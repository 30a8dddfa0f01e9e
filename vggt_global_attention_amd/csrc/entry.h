// Host-side checks and the block runner shared by the C entry points
// (api.cpp) and the layer schedule (schedule.cpp).
#pragma once

#include "plan.h"

namespace vggt {

bool aligned(const void* ptr, uintptr_t a);
bool overlap(const void* a, size_t na, const void* b, size_t nb);

// Validates one block call (shape, pointers, alignment, aliasing, workspace)
// and fills its plan; launches nothing.
int check_call(int mode, const vggt_attn_shape* shape, const CallOpts& o, const void* X,
               const void* Wqkv, const void* Wo, const float* qg, const float* qb, const float* kg,
               const float* kb, void* Y, void* ws, size_t ws_bytes, Plan* plan);

// Checks, then enqueues stages first_stage..last_stage of one block call.
int run(int mode, const CallOpts& o, int first_stage, int last_stage,
        const vggt_attn_shape* shape, const void* X, const void* Wqkv, const void* Wo,
        const float* qg, const float* qb, const float* kg, const float* kb, void* Y, void* ws,
        size_t ws_bytes, void* stream);

// Argument checks of vggt_attn_residual (no launch).
int check_residual(const void* X, const void* Y, const void* Z, int64_t rows, int d,
                   const float* gamma, int period, int active, const void* C, int64_t c_stride);

}  // namespace vggt
