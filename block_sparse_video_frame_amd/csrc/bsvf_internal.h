// Internal helpers shared by the host code and the kernel launchers of the
// bsvf library.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "bsvf.h"

namespace bsvf {

// Records a message for attn_last_error() and returns `status`.
int fail(int status, const std::string& msg);
// Clears the per-thread message and returns ATTN_OK.
int ok();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks one bf16 [B][H][N][D] tensor description: non-NULL, 16-byte aligned
// base, strides positive multiples of 8 elements (16 bytes), rows of D
// elements do not overlap within a head, and a head's span fits in int32
// element offsets from the head base.
int check_tensor(const char* name, const void* p, const int64_t* s,
                 int32_t B, int32_t H, int32_t N, int32_t D);

// Enqueues head_max[bh] = (max_n q_norm[bh][n], max_g k_gmax[bh][g]) for the
// `bh` (batch, head) pairs of contiguous fp32 norms over `n` rows (n % 16 == 0);
// bh <= 65535.  It merges into head_max with atomic maxima, so the kernel that
// wrote the norms must have set head_max to zero.  Defined with attn_norms;
// the producer uses it too.
int launch_head_max(const float* q_norm, const float* k_gmax, int32_t bh, int32_t n, float* head_max,
                    hipStream_t stream);

}  // namespace bsvf
