// attn_bwd.hip -- launch planning and dispatch of the backward kernels
// (attn_bwd_kernel.hpp).  Built as its own object: these kernels keep their
// MFMA accumulators in AGPRs where the register allocator wants them.
#include "attn_bwd_kernel.hpp"

namespace attn {

namespace {

template <int D>
BwdPlan plan_of() {
  using C = bwd::BwdCfg<D>;
  BwdPlan p;
  p.dkdv_keys_per_workgroup = C::BN;
  p.dkdv_query_step = C::STEP;
  p.dq_queries_per_workgroup = C::BM;
  p.dq_key_step = C::STEP;
  p.threads_per_workgroup = C::NT;
  p.lds_bytes = C::LDS_BYTES;
  return p;
}

template <int D, bool CAUSAL, int DT>
hipError_t launch(BwdProblem p, hipStream_t st) {
  using C = bwd::BwdCfg<D>;
  // the dQ kernel writes D_i, which the dK/dV kernel reads
  if (p.Sq > 0 && p.BH > 0)
    hipLaunchKernelGGL((bwd::attn_bwd_dq<D, CAUSAL, DT>), dim3((unsigned)(p.BH * p.nq)), dim3(C::NT), 0, st, p);
  if (p.Skv > 0 && p.BH > 0)
    hipLaunchKernelGGL((bwd::attn_bwd_dkdv<D, CAUSAL, DT>), dim3((unsigned)(p.BH * p.nk)), dim3(C::NT), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch(BwdProblem p, bool causal, int dtype, hipStream_t st) {
  using C = bwd::BwdCfg<D>;
  p.nq = (p.Sq + C::BM - 1) / C::BM;
  p.nk = (p.Skv + C::BN - 1) / C::BN;
  p.map_q = make_tile_map(p.BH * p.nq, p.nq, causal, p.hchunk_q);
  p.map_k = make_tile_map(p.BH * p.nk, p.nk, causal, p.hchunk_k);
  if (dtype == DT_F16)
    return causal ? launch<D, true, DT_F16>(p, st) : launch<D, false, DT_F16>(p, st);
  return causal ? launch<D, true, DT_BF16>(p, st) : launch<D, false, DT_BF16>(p, st);
}

}  // namespace

BwdPlan bwd_plan(int D) {
  switch (D) {
    case 64: return plan_of<64>();
    case 128: return plan_of<128>();
    default: return plan_of<256>();
  }
}

hipError_t bwd_launch(BwdProblem p, int D, bool causal, int dtype, hipStream_t stream) {
  switch (D) {
    case 64: return dispatch<64>(p, causal, dtype, stream);
    case 128: return dispatch<128>(p, causal, dtype, stream);
    default: return dispatch<256>(p, causal, dtype, stream);
  }
}

}  // namespace attn
