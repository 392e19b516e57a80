/*
 * attn_unfused.h -- C ABI of libattn_unfused.so, the unfused attention
 * forward: a comparator for the fused kernels of libattn.so (attn.h) that
 * sends the S x S score matrix through memory.  It is a library of its own so
 * that the fused library links no vendor BLAS.
 *
 * Shapes, dtypes, status codes and the causal and LSE conventions are those
 * of attn.h.  Argument checks happen before any HIP call and return a status
 * code; nothing is thrown.
 */
#ifndef EXACT_ATTENTION_52_AMD_ATTN_UNFUSED_H
#define EXACT_ATTENTION_52_AMD_ATTN_UNFUSED_H

#include <stdint.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_fwd_unfused -- the same forward as attn_fwd, unfused: a comparator
 * that shows the HBM traffic the fused kernels avoid.
 *
 * Steps: S = scale Q K^T as fp32 into the workspace (vendor strided-batched
 * GEMM over the B*H heads, the batched 4-D GEMM of the docs.rs page
 * "aprender-train 0.36.0, entrenar/autograd/cuda_forward/matmul.rs",
 * batched_4d_gemm_forward); a row softmax kernel writing the unnormalised P
 * (against the exact row max) rounded to `dtype`, the LSE and 1 / (fp32 sum
 * of P); O = P V (vendor GEMM, fp32 accumulation), then scaled by that factor
 * and rounded.  Per head S*S*12 bytes go through HBM.
 *
 *   q, k, v, o, lse, B, H, S, D, scale, causal, dtype, stream: as attn_fwd.
 *   workspace        device memory of at least
 *                    attn_fwd_unfused_workspace_bytes(B, H, S, D) bytes,
 *                    16-byte aligned, owned by the caller, overwritten; must
 *                    not overlap q, k, v, o or lse.
 *   workspace_bytes  its size.
 * Returns as attn_fwd; ATTN_ERR_BAD_ARGUMENT if the workspace is too small.
 * Calls on one device are serialised on a vendor-library handle per device,
 * which this library creates on first use (its one allocation outside the
 * caller's control).  attn_unfused_last_error() gives the text of the last
 * failure on the calling thread.
 */
int attn_fwd_unfused(const void* q, const void* k, const void* v, void* o,
                     float* lse, void* workspace, int64_t workspace_bytes,
                     int64_t B, int64_t H, int64_t S, int64_t D, float scale,
                     int causal, int dtype, void* stream);

/* Workspace bytes attn_fwd_unfused needs (per head S rows of fp32 scores
 * and of 16-bit probabilities, rows padded to 16 bytes, plus the fp32 output
 * before normalisation and one fp32 factor per row); -1 for negative or
 * overflowing sizes or an unsupported head dim. */
int64_t attn_fwd_unfused_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D);

/* Text of the last failure of an attn_fwd_unfused call on the calling thread
 * (empty after a success). */
const char* attn_unfused_last_error(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* EXACT_ATTENTION_52_AMD_ATTN_UNFUSED_H */
