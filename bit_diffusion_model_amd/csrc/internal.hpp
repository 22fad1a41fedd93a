// Internal helpers shared by the C ABI translation units (host code only).
#pragma once
#include <stdint.h>

#include "../../include/svdq.h"

namespace svdq {

// Record a failure message (thread-local) and return st.
svdq_status fail(svdq_status st, const char* fmt, ...);
// Clear the message and return SVDQ_OK.
svdq_status ok();
// Validate K, N, fmt (K a positive multiple of 128, N >= 1, known format).
svdq_status check_dims(int64_t K, int64_t N, int32_t fmt);
int group_of(int fmt);
// svdq_linear_forward's body (the caller's workspace of ws_bytes bytes, device memory).
svdq_status linear_forward(const svdq_layer* layer, int64_t M, const uint16_t* X, int64_t ldx, void* Y, int64_t ldy,
                           int32_t ydtype, void* workspace, size_t ws_bytes, void* stream);

}  // namespace svdq
