/*
 * attn.h -- C ABI of the MI355X (gfx950) exact attention library.
 *
 * The operation is the fused, tiled, exact scaled-dot-product attention of
 * the docs.rs page "oxicuda-dnn 0.1.8, src/attn/flash_attn/hopper.rs":
 *   forward (doc comment of FlashAttention3Plan::generate_forward): scores
 *   S = Q K^T scaled by the softmax scale, future positions removed when
 *   causal, an online softmax with a running max m and running sum l,
 *   O = (P V) / l, and the per-row log-sum-exp m + log(l); the S x S score
 *   matrix never reaches memory;
 *   backward (doc comment of generate_backward): dQ, dK, dV recomputing P
 *   from the saved log-sum-exp.
 *
 * Entry points: attn_fwd (contiguous), attn_fwd_strided (strides, Sq != Skv),
 * attn_bwd / attn_bwd_strided / attn_bwd_noalloc (backward), attn_fwd_variant (other copy
 * schedules, for A/B measurements), and host-only planning helpers.  The
 * unfused comparator (attn_fwd_unfused) is in its own library, declared in
 * attn_unfused.h.
 *
 * Conventions shared by every entry point:
 *   - Q, K, V, O (and dQ, dK, dV, dO) are [B, H, rows, D] of 16-bit elements
 *     (fp16 or bf16, chosen by `dtype`), contiguous C order unless an entry
 *     point takes strides; LSE (and D_i) are [B, H, Sq] fp32, contiguous.
 *   - The caller owns every buffer and the library keeps no pointer from a
 *     call.  The kernels use no memory beyond the caller's buffers, and the
 *     library allocates nothing.
 *   - Causal keeps key j for query i iff j <= i + (Skv - Sq): j <= i when
 *     Sq == Skv, and in general the last query sees the last key.
 *   - LSE is the natural logarithm of sum_j exp(scale * q_i . k_j) over the
 *     kept keys.
 *   - Status codes are returned, never thrown; attn_last_error() gives a
 *     thread-local text for the most recent failure on the calling thread.
 *   - All argument checks happen before any HIP call.  A failed check
 *     launches nothing and leaves every output untouched.
 */
#ifndef EXACT_ATTENTION_52_AMD_ATTN_H
#define EXACT_ATTENTION_52_AMD_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 6

/* Element type of Q, K, V and O.  The page's configuration check
 * (validate_config of FlashAttention3Config) accepts only the two 16-bit
 * float types. */
typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL_PTR = 1,              /* a required pointer is NULL          */
  ATTN_ERR_BAD_SHAPE = 2,             /* B, H or S < 0, or sizes overflow    */
  ATTN_ERR_UNSUPPORTED_HEAD_DIM = 3,  /* D not in {64, 128, 256}             */
  ATTN_ERR_UNSUPPORTED_DTYPE = 4,     /* dtype not ATTN_F16 / ATTN_BF16      */
  ATTN_ERR_MISALIGNED = 5,            /* q/k/v/o not 16-B, lse not 4-B       */
  ATTN_ERR_BAD_SCALE = 6,             /* scale NaN or infinite               */
  ATTN_ERR_ALIASING = 7,              /* an output overlaps another buffer   */
  ATTN_ERR_UNSUPPORTED_DEVICE = 8,    /* current device is not gfx950        */
  ATTN_ERR_LAUNCH = 9,                /* the HIP runtime refused the launch  */
  ATTN_ERR_BAD_ARGUMENT = 10          /* any other invalid argument          */
} attn_status_t;

/*
 * attn_fwd -- O = softmax(scale * Q K^T [+ causal mask]) V and LSE.
 *
 * Defined by the doc comment of FlashAttention3Plan::generate_forward on the
 * page named above (Q K^T, online softmax with running max and sum, optional
 * causal removal of future positions, O = O_acc / l, LSE = m + log(l)); its
 * kernel parameters (q, k, v, o, lse pointers, sequence length, head_dim,
 * num_heads, sm_scale) are the ones taken here, with batch and heads as
 * explicit sizes instead of strides.
 *
 *   q, k, v  device pointers, [B,H,S,D] `dtype` elements, read only; they may
 *            alias one another.  16-byte aligned.
 *   o        device pointer, [B,H,S,D] `dtype`, written in full (each element
 *            rounded to nearest-even from the fp32 result).  16-byte aligned;
 *            must not overlap q, k, v or lse.
 *   lse      device pointer, [B,H,S] fp32, written in full.  4-byte aligned;
 *            must not overlap q, k, v or o.
 *   B, H, S  batch, heads, sequence length (>= 0; any S, no multiple needed).
 *            B*H*S == 0 is a valid empty call: nothing is launched.
 *   D        head dimension: 64, 128 or 256 (the page's supported set).
 *   scale    softmax scale applied to Q K^T (the page's f32 sm_scale); any
 *            finite value (0 gives a uniform softmax over the kept keys; a
 *            negative scale is exact: it multiplies -Q by |scale|).
 *   causal   0 or 1 (any non-zero value means 1).
 *   dtype    ATTN_F16 or ATTN_BF16.
 *   stream   hipStream_t to enqueue on; NULL means the null stream.
 *
 * Returns ATTN_OK once the kernel is enqueued (asynchronous: no
 * synchronisation happens), else an attn_status_t code.  Reentrant and
 * thread-safe.  The result is deterministic: every output element is written
 * by exactly one workgroup with a fixed order of arithmetic.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t S, int64_t D, float scale,
             int causal, int dtype, void* stream);

/*
 * attn_fwd_strided -- attn_fwd for queries and keys of different lengths and
 * for strided tensors.
 *
 * The page's kernel takes separate query and key/value sequence lengths and
 * per-tensor batch/head strides (doc comment of
 * FlashAttention3Plan::generate_forward and its kernel parameter list); this
 * entry point takes both, plus row strides.
 *
 *   q        [B,H,Sq,D]  element (b,h,i,d) at q + b*qs[0] + h*qs[1] + i*qs[2] + d
 *   k, v     [B,H,Skv,D] likewise with k_strides / v_strides
 *   o        [B,H,Sq,D]  likewise with o_strides (written in full)
 *   lse      [B,H,Sq] fp32, contiguous (written in full)
 *   *_strides  host arrays of 3 int64 (batch, head, row strides in elements)
 *              or NULL for contiguous [B,H,rows,D].  Every stride of a
 *              dimension longer than 1 must be a multiple of 8 elements
 *              (16 bytes) and >= 0; row strides >= D; o's strides must not
 *              make two elements share an address; one head of any tensor
 *              must span less than 2 GiB.
 *   Sq, Skv  >= 0.  B*H*Sq == 0 is a valid empty call.  With Skv == 0 no
 *            key is read and k, v may be NULL.
 *   causal   keeps key j for query i iff j <= i + (Skv - Sq): the last query
 *            sees the last key (j <= i when Sq == Skv).  A query with no key
 *            left (causal, Sq > Skv; or Skv == 0) gets O = 0 and LSE = -inf.
 * Everything else (pointer alignment, dtype, head dim, scale, aliasing,
 * stream, errors) is as for attn_fwd; aliasing is judged on each tensor's
 * byte extent from its first to its last element.
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                     const int64_t* q_strides, const int64_t* k_strides,
                     const int64_t* v_strides, const int64_t* o_strides, float scale,
                     int causal, int dtype, void* stream);

/*
 * attn_bwd -- gradients of the attention forward for a given dO.
 *
 * The page's backward (doc comment of FlashAttention3Plan::generate_backward)
 * recomputes P from the saved log-sum-exp and forms dV = P^T dO,
 * dP = dO V^T, dS = P * (dP - D_i) with D_i = rowsum(dO * O), dQ = dS K and
 * dK = dS^T Q; its kernel takes q, k, v, o, do, lse, di, dq, dk, dv, the
 * query and key/value lengths and sm_scale, as this call does.  dS is the
 * gradient of the scaled scores, so dQ and dK carry the factor `scale`.
 * dQ is accumulated without atomics: one kernel per key tile writes dK, dV,
 * another per query tile writes dQ, so the result is deterministic.
 *
 *   q, o, dO  [B,H,Sq,D] `dtype`, contiguous, read only (o and lse as the
 *             forward returned them for the same q, k, v, scale, causal)
 *   k, v      [B,H,Skv,D] `dtype`, contiguous, read only
 *   lse       [B,H,Sq] fp32 natural-log LSE from the forward, read only
 *   dq        [B,H,Sq,D] `dtype`, written in full
 *   dk, dv    [B,H,Skv,D] `dtype`, written in full
 *   delta     [B,H,Sq] fp32, written in full with D_i (the page's di)
 *   Sq, Skv   >= 0; causal keeps key j for query i iff j <= i + (Skv - Sq),
 *             as in attn_fwd_strided.  Keys no query sees get dK = dV = 0,
 *             queries with no key dQ = 0 and D_i = 0.
 *   D, scale, causal, dtype, stream   as for attn_fwd.
 * Inputs may alias one another; dq, dk, dv and delta must not overlap each
 * other or any input.  16-bit tensors 16-byte aligned, fp32 ones 4-byte.
 * Pointers of tensors with no element (Sq == 0: q, o, dO, lse, dq, delta;
 * Skv == 0: k, v, dk, dv) may be NULL.  B*H == 0, or Sq == Skv == 0, is a
 * valid empty call.  Errors and asynchrony as for attn_fwd.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dO, void* dq, void* dk, void* dv,
             float* delta, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
             int64_t D, float scale, int causal, int dtype, void* stream);

/*
 * attn_bwd_strided -- attn_bwd for strided tensors.
 *
 * Same operation, results and errors as attn_bwd; every 16-bit tensor takes
 * a host array of 3 int64 (batch, head, row) strides in elements, or NULL
 * for contiguous [B,H,rows,D], under the rules of attn_fwd_strided (strides
 * of dimensions longer than 1 >= 0 and multiples of 8, row strides >= D, one
 * head < 2 GiB; dq, dk and dv must not address one element twice).  lse and
 * delta stay contiguous [B,H,Sq].  Aliasing is judged on byte extents.
 */
int attn_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dO, void* dq, void* dk, void* dv,
                     float* delta, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                     int64_t D, const int64_t* q_strides, const int64_t* k_strides,
                     const int64_t* v_strides, const int64_t* o_strides,
                     const int64_t* do_strides, const int64_t* dq_strides,
                     const int64_t* dk_strides, const int64_t* dv_strides, float scale,
                     int causal, int dtype, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd that allocates nothing and takes no
 * workspace, for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, checks, results and errors as attn_bwd, except that D_i
 * (attn_bwd's `delta`) is not returned: it lives in a file-scope device
 * array of the library, 16 MiB per GPU (2^22 fp32 rows), held from the
 * library's load until the process ends.  B*H*Sq above 2^22 returns
 * ATTN_ERR_BAD_ARGUMENT before any HIP call.  The array's address on the
 * current device is looked up once per device (hipGetSymbolAddress); after
 * that no call makes a runtime allocation.  Every call on a GPU shares that
 * GPU's array: calls that overlap in time on one GPU (different streams,
 * threads or processes sharing a context) race on D_i and must be
 * serialised by the caller.  Each call writes every D_i it reads before
 * reading it, so nothing needs clearing between calls.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dO, void* dq, void* dk, void* dv,
                     int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                     float scale, int causal, int dtype, void* stream);

/*
 * attn_fwd_variant -- attn_fwd with another copy schedule, for A/B
 * measurements of the pipeline depth and of a producer/consumer wave split
 * (the page's FlashAttention3Config makes pingpong_stages and
 * num_producer_warps first-class knobs).  Arguments, checks, results
 * contract and errors as attn_fwd; `variant`:
 *   0  the shipped configuration (identical to attn_fwd)
 *   1  1 K/V stage in LDS: copy tile j, wait, compute it
 *   2  2 stages: tile j+1 copied while tile j is computed
 *   3  3 stages: tile j+2 copied while tile j is computed
 *   4  2 stages and one extra producer wave that issues every HBM -> LDS
 *      copy while the other waves only compute
 *   5  the shipped tile shape of the head dim, 1 stage, one wave step after
 *      another (no ping-pong of wave groups, no staggered copies, no in-wave
 *      pipeline; at D = 256 the shape attn_fwd picks for these sizes)
 *   6  the shipped tile shape of the head dim, 2 stages, one barrier per tile
 * Variants 1-4 exist for D = 64 (the shipped 4-wave, 64-key tile shape, so
 * variant 2 is attn_fwd itself) and D = 128 (4 computing waves, 64-key
 * tiles, so that 3 stages fit); variants 5 and 6 for every head dim.  Others
 * return ATTN_ERR_BAD_ARGUMENT.  Every variant's waves run the same per-wave
 * arithmetic in the same order as the shipped kernel of their tile shape, so
 * variants 5 and 6 (and 1-4 at D = 64) are bit-identical to attn_fwd, and
 * 1-4 to one another: a race in any schedule shows up as a difference.
 */
int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t S, int64_t D, float scale,
                     int causal, int dtype, int variant, void* stream);

/*
 * attn_fwd_plan -- the launch geometry attn_fwd would use (host only, no HIP
 * call, no device needed).  Mirrors the page's launch_params: one workgroup
 * per (query tile, batch*head), num_q_tiles = ceil(S / block_m); the key
 * length changes the loop trip count, not the grid.  block_m is 128 at D=64,
 * 256 at D=128; at D=256 it is 128 where B*H*ceil(S/128) >= 512 (the
 * in-wave pipelined kernel) and 64 otherwise.
 */
typedef struct {
  int64_t block_m;               /* query rows per workgroup               */
  int64_t block_n;               /* keys per K/V tile                      */
  int64_t kv_stages;             /* LDS buffers for K/V tiles              */
  int64_t waves_q;               /* waves splitting the query rows         */
  int64_t waves_k;               /* waves splitting each key tile          */
  int64_t threads_per_workgroup; /* 64 * waves_q * waves_k                 */
  int64_t lds_bytes;             /* LDS per workgroup                      */
  int64_t num_q_tiles;           /* ceil(S / block_m)                      */
  int64_t num_workgroups;        /* num_q_tiles * B * H                    */
} attn_fwd_plan_t;

/* Returns ATTN_OK and fills *out, or a status code for invalid sizes,
 * head dim or dtype (same rules as attn_fwd), or ATTN_ERR_NULL_PTR. */
int attn_fwd_plan(int64_t B, int64_t H, int64_t S, int64_t D, int causal,
                  int dtype, attn_fwd_plan_t* out);

/*
 * attn_fwd_workgroup_tile -- which (query tile, b*H + h) the workgroup with
 * linear id `wg` (0 <= wg < num_workgroups) computes (host only).  The map is
 * a bijection.  Non-causal: each XCD (workgroup id mod 8) gets a contiguous run
 * of heads.  Causal: ids go in order of decreasing cost (last query tile of
 * every head first), so each XCD runs its share longest first; when B*H is a
 * multiple of 8, head h stays on XCD h mod 8.
 */
int attn_fwd_workgroup_tile(int64_t B, int64_t H, int64_t S, int64_t D,
                            int causal, int dtype, int64_t wg,
                            int64_t* q_tile, int64_t* bh);

/* Static text for a status code ("unknown status" for others). */
const char* attn_status_string(int status);

/* Detail of the last non-OK return on this thread ("" if none). */
const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the loaded library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_52_AMD_ATTN_H */
