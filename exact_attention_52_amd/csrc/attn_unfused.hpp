// attn_unfused.hpp -- host-side view of the unfused comparator
// (attn_unfused.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Workspace layout (each part 256-byte aligned): S as fp32 rows ld_s apart;
// P in the input dtype, rows ld_p apart; O before normalisation, fp32
// [B,H,S,D]; per row 1 / (fp32 sum of P), fp32.
struct UnfusedLayout {
  int64_t ld_s, ld_p;  // elements
  int64_t s_bytes, p_offset, o_offset, r_offset, bytes;
};

UnfusedLayout unfused_layout(int64_t B, int64_t H, int64_t S, int64_t D);

// Enqueue S = scale Q K^T, the row softmax and O = P V on `stream`; nullptr on
// success, else a static description of what failed.  Arguments validated by
// the caller; q, k, v, o contiguous [B,H,S,D]; ws at least unfused_layout().bytes.
const char* unfused_launch(const void* q, const void* k, const void* v, void* o, float* lse, void* ws, int64_t B,
                           int64_t H, int64_t S, int64_t D, float scale, bool causal, int dtype,
                           hipStream_t stream);

}  // namespace attn
