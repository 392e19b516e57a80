// attn_variants.hip -- schedule variants of kernel 1 for A/B measurements of
// the K/V pipeline depth and of a producer/consumer wave split (the page's
// Hopper design makes both first-class knobs: pingpong_stages and
// num_producer_warps of FlashAttention3Config).  Same computation and
// results contract as attn_fwd; only the copy schedule differs:
//   1: 1 LDS stage   (copy tile j, wait, compute tile j, wait)
//   2: 2 LDS stages  (copy tile j+1 while computing tile j)
//   3: 3 LDS stages  (copy tile j+2 while computing tile j; counted waits)
//   4: 2 LDS stages, plus one producer wave that issues every HBM -> LDS copy
//      while the other waves only compute
// D=64: 8 computing waves x 32 query rows, 128-key tiles (one workgroup per
// CU; attn_fwd itself runs 4-wave, 128-row workgroups at D=64, two per CU);
// D=128: 4 computing waves, 64-key tiles (so that 3 stages fit).
#include "attn_variants.hpp"

namespace attn {
namespace {

template <int D, int S, bool P>
using V64 = TileCfg<64, 8, 1, 128, false, false, S, P>;
template <int D, int S, bool P>
using V128 = TileCfg<128, 4, 1, 64, false, false, S, P>;

template <class C, bool CAUSAL, int DT>
hipError_t go(Problem p, hipStream_t st) {
  p.nq = (p.Sq + C::BM - 1) / C::BM;
  const int64_t BH = p.G;  // the caller passes B*H here
  p.G = (int64_t)p.nq * BH;
  if (p.G > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_kernel<C, CAUSAL, DT>), dim3((unsigned)p.G), dim3(C::NT), 0, st, p);
  return hipGetLastError();
}

template <class C>
hipError_t pick(const Problem& p, bool causal, int dtype, hipStream_t st) {
  if (dtype == DT_F16) return causal ? go<C, true, DT_F16>(p, st) : go<C, false, DT_F16>(p, st);
  return causal ? go<C, true, DT_BF16>(p, st) : go<C, false, DT_BF16>(p, st);
}

template <int D, template <int, int, bool> class V>
hipError_t by_variant(const Problem& p, bool causal, int dtype, int v, hipStream_t st) {
  switch (v) {
    case 1: return pick<V<D, 1, false>>(p, causal, dtype, st);
    case 2: return pick<V<D, 2, false>>(p, causal, dtype, st);
    case 3: return pick<V<D, 3, false>>(p, causal, dtype, st);
    case 4: return pick<V<D, 2, true>>(p, causal, dtype, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int variant_block_m(int D, int v) {
  if (v < 1 || v >= kNumVariants) return 0;
  if (D == 64) return V64<64, 2, false>::BM;
  if (D == 128) return V128<128, 2, false>::BM;
  return 0;
}

hipError_t variant_launch(Problem p, int D, bool causal, int dtype, int v, hipStream_t stream) {
  if (D == 64) return by_variant<64, V64>(p, causal, dtype, v, stream);
  if (D == 128) return by_variant<128, V128>(p, causal, dtype, v, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
