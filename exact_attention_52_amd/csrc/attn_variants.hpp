// attn_variants.hpp -- schedule variants of the forward kernel for A/B
// measurements (attn_variants.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_fwd_kernel.hpp"

namespace attn {

constexpr int kNumVariants = 7;  // 0 is the shipped configuration

// Launch variant v (1..kNumVariants-1) for head dim D on `p`, setting
// p.nq and p.G for the variant's query tile.  Returns hipErrorInvalidValue
// for an unsupported (v, D) or a grid over the launch limit.
hipError_t variant_launch(Problem p, int D, bool causal, int dtype, int v, hipStream_t stream);

// Query rows per workgroup of variant v at head dim D for BH heads of S
// query rows (0 if unsupported).
int variant_block_m(int D, int v, int64_t BH, int64_t S);

}  // namespace attn
