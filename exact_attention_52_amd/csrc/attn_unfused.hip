// attn_unfused.hip -- the unfused attention forward, as a comparator for the
// fused kernels: the score matrix goes through HBM.
//
//   1. S = scale * Q K^T for every (b, h), fp32, written to a workspace
//      (rocBLAS strided-batched GEMM over the B*H heads);
//   2. one workgroup per row: mask, row max, P = exp(s - m) rounded to the
//      input dtype, LSE = m + log l, and 1 / l, l the fp32 sum of P;
//   3. O = P V (rocBLAS strided-batched GEMM, fp32 accumulation and output);
//   4. O times that factor per row, rounded to the input dtype.
// P is taken against the exact row max, so the row's largest P is exp(0) =
// 1, exact in 16 bits, and O normalised by the fp32 sum then carries only the
// other keys' 16-bit rounding, weighted by their (small) P.  Rounding the
// normalised P instead moves a peaky fp16 row by up to u/2 of its largest V
// entries; normalising by the sum of the rounded P multiplies the other keys'
// rounding by V_j - O, which reached 2.03e-3 (over the 2e-3 fp16 bound) on a
// peaky row with |O| ~ 4.5.
// The batched 4-D GEMM of the docs.rs page "aprender-train 0.36.0,
// entrenar/autograd/cuda_forward/matmul.rs" (doc comment of
// batched_4d_gemm_forward: C[b,h] = A[b,h] B[b,h] over [batch, heads, m, k]
// and [batch, heads, k, n]) is exactly the contraction of steps 1 and 3.  Per
// head it moves S*S*(4 + 4 + 2 + 2) bytes through HBM (write S, read S,
// write P, read P) that the fused kernels keep on chip.
//
// This file is all of libattn_unfused.so, a library of its own: the fused
// library libattn.so links no vendor BLAS.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <cmath>
#include <mutex>
#include <unordered_map>

#include "attn_common.hpp"
#include "attn_unfused.h"
#include "attn_unfused.hpp"

namespace attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == 0) {
    f16x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  } else {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
}

// Workgroup-wide reduction of one float (max or sum) through LDS.
template <bool MAX>
__device__ __forceinline__ float block_reduce(float x, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m /= 2) {
    const float y = __shfl_xor(x, m, 64);
    x = MAX ? fmaxf(x, y) : x + y;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red is reused between calls
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  x = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) x = MAX ? fmaxf(x, red[w]) : x + red[w];
  return x;
}

// One workgroup per score row (b*H + h)*S + i.  The row (ld floats apart,
// Skv valid) is read once into registers when NC > 0 (NC float4 chunks per
// thread, Skv <= 1024*NC) or streamed twice when NC == 0.  Keys past the end
// or after the query (causal) get P = 0; a row with no key gets LSE = -inf.
template <int NC, int DT>
__global__ __launch_bounds__(kThreads) void row_softmax(const float* __restrict__ s, uint16_t* __restrict__ p,
                                                        float* __restrict__ lse, float* __restrict__ inv_l, int S,
                                                        int64_t ld_s, int64_t ld_p, int causal) {
  __shared__ float red[kThreads / 64];
  const int64_t row = blockIdx.x;
  const int i = (int)(row % S);
  const int kept = causal ? i + 1 : S;  // keys 0 .. kept-1
  const float* srow = s + row * ld_s;
  uint16_t* prow = p + row * ld_p;
  constexpr float kLog2e = 1.4426950408889634074f;
  const int nchunk = (S + 3) / 4;

  auto val = [&](const f32x4& x, int c, int e) __attribute__((always_inline)) {
    return 4 * c + e < kept ? x[e] : -__builtin_inff();
  };
  float m = -__builtin_inff();
  f32x4 xs[NC > 0 ? NC : 1];
  if constexpr (NC > 0) {
#pragma unroll
    for (int r = 0; r < NC; ++r) {
      const int c = threadIdx.x + kThreads * r;
      xs[r] = c < nchunk ? *reinterpret_cast<const f32x4*>(srow + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, c < nchunk ? val(xs[r], c, e) : -__builtin_inff());
    }
  } else {
    for (int c = threadIdx.x; c < nchunk; c += kThreads) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(srow + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, val(x, c, e));
    }
  }
  m = block_reduce<true>(m, red);
  // exp2 offset: 0 for a row with no key (every value is -inf, P = 0)
  const float off = m == -__builtin_inff() ? 0.f : -m * kLog2e;
  // l: fp32 sum of P (the LSE and O's normaliser)
  float l = 0.f;
  auto store = [&](const f32x4& pe, int c) __attribute__((always_inline)) {
    const u32x2 w = {pack2<DT>(pe[0], pe[1]), pack2<DT>(pe[2], pe[3])};
    *reinterpret_cast<u32x2*>(prow + 4 * c) = w;
  };
  auto expo = [&](f32x4 x, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(val(x, c, e), kLog2e, off));
      l += x[e];
    }
    return x;
  };
  if constexpr (NC > 0) {
#pragma unroll
    for (int r = 0; r < NC; ++r) {
      const int c = threadIdx.x + kThreads * r;
      if (c < nchunk) store(expo(xs[r], c), c);
    }
  } else {
    for (int c = threadIdx.x; c < nchunk; c += kThreads) store(expo(*reinterpret_cast<const f32x4*>(srow + 4 * c), c), c);
  }
  l = block_reduce<false>(l, red);
  if (threadIdx.x == 0) {
    lse[row] = l > 0.f ? m + __builtin_amdgcn_logf(l) * 0.69314718055994530942f : -__builtin_inff();
    inv_l[row] = l > 0.f ? 1.f / l : 0.f;
  }
}

// O = O32 * inv_l per row, rounded to the input dtype; 8 elements a thread.
template <int DT>
__global__ __launch_bounds__(kThreads) void scale_rows(const float* __restrict__ o32, const float* __restrict__ inv_l,
                                                       uint16_t* __restrict__ o, int64_t n8, int D) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= n8) return;
  const float f = inv_l[t * 8 / D];
  const f32x4 a = *reinterpret_cast<const f32x4*>(o32 + 8 * t);
  const f32x4 b = *reinterpret_cast<const f32x4*>(o32 + 8 * t + 4);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {pack2<DT>(a[0] * f, a[1] * f), pack2<DT>(a[2] * f, a[3] * f), pack2<DT>(b[0] * f, b[1] * f),
                   pack2<DT>(b[2] * f, b[3] * f)};
  *reinterpret_cast<u32x4*>(o + 8 * t) = w;
}

// One rocBLAS handle per device, created on first use; calls that enqueue
// on it are serialised (the handle's stream is set per call).
std::mutex g_blas_mutex;
std::unordered_map<int, rocblas_handle> g_handles;

}  // namespace

UnfusedLayout unfused_layout(int64_t B, int64_t H, int64_t S, int64_t D) {
  UnfusedLayout u;
  u.ld_s = (S + 3) / 4 * 4;  // fp32 rows start 16-byte aligned
  u.ld_p = (S + 7) / 8 * 8;  // 16-bit rows start 16-byte aligned
  u.s_bytes = B * H * S * u.ld_s * 4;
  u.p_offset = (u.s_bytes + 255) / 256 * 256;
  u.o_offset = (u.p_offset + B * H * S * u.ld_p * 2 + 255) / 256 * 256;
  u.r_offset = u.o_offset + B * H * S * D * 4;
  u.bytes = u.r_offset + B * H * S * 4;
  return u;
}

const char* unfused_launch(const void* q, const void* k, const void* v, void* o, float* lse, void* ws, int64_t B,
                           int64_t H, int64_t S, int64_t D, float scale, bool causal, int dtype,
                           hipStream_t stream) {
  const UnfusedLayout u = unfused_layout(B, H, S, D);
  float* sbuf = static_cast<float*>(ws);
  uint16_t* pbuf = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + u.p_offset);
  float* o32 = reinterpret_cast<float*>(static_cast<char*>(ws) + u.o_offset);
  float* inv_l = reinterpret_cast<float*>(static_cast<char*>(ws) + u.r_offset);
  const rocblas_datatype in_t = dtype == 0 ? rocblas_datatype_f16_r : rocblas_datatype_bf16_r;
  const int batch = (int)(B * H);
  {
    std::lock_guard<std::mutex> lock(g_blas_mutex);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return "hipGetDevice failed";
    rocblas_handle& h = g_handles[dev];
    if (!h && rocblas_create_handle(&h) != rocblas_status_success) {
      h = nullptr;
      return "rocblas_create_handle failed";
    }
    if (rocblas_set_stream(h, stream) != rocblas_status_success) return "rocblas_set_stream failed";
    // column-major view: row-major K [S,D] is D x S; C = K^T-op x Q is the
    // S x S column-major matrix whose memory is row-major S[i][j] (ld_s)
    const float alpha = scale, one = 1.f, beta = 0.f;
    rocblas_status st = rocblas_gemm_strided_batched_ex(
        h, rocblas_operation_transpose, rocblas_operation_none, (int)S, (int)S, (int)D, &alpha, k, in_t, (int)D,
        S * D, q, in_t, (int)D, S * D, &beta, sbuf, rocblas_datatype_f32_r, (int)u.ld_s, S * u.ld_s, sbuf,
        rocblas_datatype_f32_r, (int)u.ld_s, S * u.ld_s, batch, rocblas_datatype_f32_r, rocblas_gemm_algo_standard,
        0, 0);
    if (st != rocblas_status_success) return rocblas_status_to_string(st);
    const int64_t rows = B * H * S;
    const int nc = (int)((S + 4 * kThreads - 1) / (4 * kThreads));
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3((unsigned)rows), dim3(kThreads), 0, stream, sbuf, pbuf, lse, inv_l, (int)S,
                         u.ld_s, u.ld_p, (int)causal);
    };
    if (dtype == 0) {
      if (nc <= 1) go(row_softmax<1, 0>);
      else if (nc <= 2) go(row_softmax<2, 0>);
      else if (nc <= 4) go(row_softmax<4, 0>);
      else if (nc <= 8) go(row_softmax<8, 0>);
      else go(row_softmax<0, 0>);
    } else {
      if (nc <= 1) go(row_softmax<1, 1>);
      else if (nc <= 2) go(row_softmax<2, 1>);
      else if (nc <= 4) go(row_softmax<4, 1>);
      else if (nc <= 8) go(row_softmax<8, 1>);
      else go(row_softmax<0, 1>);
    }
    if (hipGetLastError() != hipSuccess) return "softmax kernel launch failed";
    // O^T (D x S column-major = row-major O) = V^T (D x S) x P^T (S x S)
    st = rocblas_gemm_strided_batched_ex(h, rocblas_operation_none, rocblas_operation_none, (int)D, (int)S, (int)S,
                                         &one, v, in_t, (int)D, S * D, pbuf, in_t,
                                         (int)u.ld_p, S * u.ld_p, &beta, o32, rocblas_datatype_f32_r, (int)D, S * D,
                                         o32, rocblas_datatype_f32_r, (int)D, S * D, batch, rocblas_datatype_f32_r,
                                         rocblas_gemm_algo_standard, 0, 0);
    if (st != rocblas_status_success) return rocblas_status_to_string(st);
    const int64_t n8 = B * H * S * D / 8;
    const unsigned g = (unsigned)((n8 + kThreads - 1) / kThreads);
    if (dtype == 0)
      hipLaunchKernelGGL(scale_rows<0>, dim3(g), dim3(kThreads), 0, stream, o32, inv_l, (uint16_t*)o, n8, (int)D);
    else
      hipLaunchKernelGGL(scale_rows<1>, dim3(g), dim3(kThreads), 0, stream, o32, inv_l, (uint16_t*)o, n8, (int)D);
    if (hipGetLastError() != hipSuccess) return "row scaling kernel launch failed";
  }
  return nullptr;
}

}  // namespace attn

extern "C" {

int64_t attn_fwd_unfused_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D) {
  if (B < 0 || H < 0 || S < 0 || (D != 64 && D != 128 && D != 256)) return -1;
  if (B == 0 || H == 0 || S == 0) return 0;
  // B*H*S*(S+8+D+1)*6 must fit in int64 with room for the rounding
  const int64_t lim = (int64_t)1 << 58;
  if (S > (1 << 28) || H > lim / B || B * H > lim / S / (S + D + 9) / 6) return -1;
  return attn::unfused_layout(B, H, S, D).bytes;
}

int attn_fwd_unfused(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                     int64_t workspace_bytes, int64_t B, int64_t H, int64_t S, int64_t D, float scale, int causal,
                     int dtype, void* stream) {
  int st = check_sizes(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale)) return fail(ATTN_ERR_BAD_SCALE, "scale must be finite (got %g)", (double)scale);
  if (B == 0 || H == 0 || S == 0) return ok();
  if (!q || !k || !v || !o || !lse || !workspace)
    return fail(ATTN_ERR_NULL_PTR, "q, k, v, o, lse and workspace must be non-NULL");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)workspace) & 15)
    return fail(ATTN_ERR_MISALIGNED, "q, k, v, o and workspace must be 16-byte aligned");
  if ((uintptr_t)lse & 3) return fail(ATTN_ERR_MISALIGNED, "lse must be 4-byte aligned");
  const int64_t need = attn_fwd_unfused_workspace_bytes(B, H, S, D);
  if (need < 0 || B * H > 0x7FFFFFFF || B * H * S > 0x7FFFFFFF)
    return fail(ATTN_ERR_BAD_SHAPE, "B=%lld H=%lld S=%lld too large for the unfused path", (long long)B,
                (long long)H, (long long)S);
  if (workspace_bytes < need)
    return fail(ATTN_ERR_BAD_ARGUMENT, "workspace of %lld bytes; %lld needed", (long long)workspace_bytes,
                (long long)need);
  const int64_t nt = B * H * S * D * 2, nl = B * H * S * 4;
  if (overlaps(o, nt, q, nt) || overlaps(o, nt, k, nt) || overlaps(o, nt, v, nt) || overlaps(o, nt, lse, nl))
    return fail(ATTN_ERR_ALIASING, "o overlaps q, k, v or lse");
  if (overlaps(lse, nl, q, nt) || overlaps(lse, nl, k, nt) || overlaps(lse, nl, v, nt))
    return fail(ATTN_ERR_ALIASING, "lse overlaps q, k or v");
  for (const void* t : {(const void*)q, (const void*)k, (const void*)v, (const void*)o})
    if (overlaps(workspace, need, t, nt)) return fail(ATTN_ERR_ALIASING, "workspace overlaps q, k, v or o");
  if (overlaps(workspace, need, lse, nl)) return fail(ATTN_ERR_ALIASING, "workspace overlaps lse");
  st = check_device();
  if (st != ATTN_OK) return st;
  const char* err = attn::unfused_launch(q, k, v, o, lse, workspace, B, H, S, D, scale, causal != 0, dtype,
                                         (hipStream_t)stream);
  if (err) return fail(ATTN_ERR_LAUNCH, "unfused path: %s", err);
  return ok();
}

const char* attn_unfused_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
