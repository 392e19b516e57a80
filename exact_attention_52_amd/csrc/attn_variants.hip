// attn_variants.hip -- schedule variants of the forward kernel, for A/B
// measurements of the K/V pipeline depth and of a producer/consumer wave
// split (the page's Hopper design makes both first-class knobs:
// pingpong_stages and num_producer_warps of FlashAttention3Config), and as a
// race canary for the shipped schedules.  Same computation and results
// contract as attn_fwd; only the copy schedule differs:
//   1: 1 LDS stage   (copy tile j, wait, compute tile j, wait)
//   2: 2 LDS stages  (copy tile j+1 while computing tile j)
//   3: 3 LDS stages  (copy tile j+2 while computing tile j; counted waits)
//   4: 2 LDS stages, plus one producer wave that issues every HBM -> LDS copy
//      while the other waves only compute
//   5: the shipped tile shape of the head dim in kernel 1 with one stage
//   6: the shipped tile shape of the head dim in kernel 1 with two stages and
//      one barrier per tile (no ping-pong, no staggered copies, no in-wave
//      pipeline)
// Variants 1-4: D=64 uses the shipped D=64 shape (4 waves x 32 query rows,
// 64-key tiles), so variant 2 is the shipped kernel itself; D=128 uses 4
// computing waves and 64-key tiles, the largest D=128 shape for which three
// stages fit in LDS.  Variants 5 and 6 exist for every head dim.  Every wave
// of every variant computes its rows with the same per-wave steps in the
// same order as the shipped kernel of its tile shape, so results are
// bit-identical to attn_fwd for the shipped shapes (variants 5, 6 and, at
// D=64, 1-4) and among variants 1-4.
#include "attn_variants.hpp"

namespace attn {
namespace {

template <int S, bool P>
using V64 = TileCfg<64, 4, 1, 64, false, false, S, P>;
template <int S, bool P>
using V128 = TileCfg<128, 4, 1, 64, false, false, S, P>;
// the shipped tile shapes (query waves, key waves, keys per tile) in kernel 1
template <int D, int S>
struct Shipped;
template <int S>
struct Shipped<64, S> {
  using C = TileCfg<64, 4, 1, 64, false, false, S>;
};
template <int S>
struct Shipped<128, S> {
  using C = TileCfg<128, 8, 1, 128, false, false, S>;
};
template <int S>
struct Shipped<256, S> {
  using C = TileCfg<256, 2, 2, 64, false, false, S>;    // grids below use_inwave_256
  using Big = TileCfg<256, 4, 1, 64, false, false, S>;  // the in-wave kernel's shape
};

template <class C, bool CAUSAL, int DT>
hipError_t go(Problem p, hipStream_t st) {
  p.nq = (p.Sq + C::BM - 1) / C::BM;
  const int64_t BH = p.G;  // the caller passes B*H here
  p.G = (int64_t)p.nq * BH;
  if (p.G > 0x7FFFFFFF) return hipErrorInvalidValue;
  p.map = make_tile_map(p.G, p.nq, CAUSAL, p.hchunk);
  hipLaunchKernelGGL((attn_fwd_kernel<C, CAUSAL, DT>), dim3((unsigned)p.G), dim3(C::NT), 0, st, p);
  return hipGetLastError();
}

template <class C>
hipError_t pick(const Problem& p, bool causal, int dtype, hipStream_t st) {
  if (dtype == DT_F16) return causal ? go<C, true, DT_F16>(p, st) : go<C, false, DT_F16>(p, st);
  return causal ? go<C, true, DT_BF16>(p, st) : go<C, false, DT_BF16>(p, st);
}

template <template <int, bool> class V>
hipError_t schedule(const Problem& p, bool causal, int dtype, int v, hipStream_t st) {
  switch (v) {
    case 1: return pick<V<1, false>>(p, causal, dtype, st);
    case 2: return pick<V<2, false>>(p, causal, dtype, st);
    case 3: return pick<V<3, false>>(p, causal, dtype, st);
    case 4: return pick<V<2, true>>(p, causal, dtype, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t shipped_shape(const Problem& p, bool causal, int dtype, int v, hipStream_t st) {
  if constexpr (D == 256) {
    if (use_inwave_256(p.G, p.Sq)) {  // p.G holds B*H here
      if (v == 5) return pick<typename Shipped<D, 1>::Big>(p, causal, dtype, st);
      return pick<typename Shipped<D, 2>::Big>(p, causal, dtype, st);
    }
  }
  if (v == 5) return pick<typename Shipped<D, 1>::C>(p, causal, dtype, st);
  return pick<typename Shipped<D, 2>::C>(p, causal, dtype, st);
}

}  // namespace

int variant_block_m(int D, int v, int64_t BH, int64_t S) {
  if (v < 1 || v >= kNumVariants) return 0;
  if (v >= 5) {
    if (D == 64) return Shipped<64, 1>::C::BM;
    if (D == 128) return Shipped<128, 1>::C::BM;
    if (D == 256) return use_inwave_256(BH, S) ? Shipped<256, 1>::Big::BM : Shipped<256, 1>::C::BM;
    return 0;
  }
  if (D == 64) return V64<2, false>::BM;
  if (D == 128) return V128<2, false>::BM;
  return 0;
}

hipError_t variant_launch(Problem p, int D, bool causal, int dtype, int v, hipStream_t stream) {
  if (v >= 5) {
    if (D == 64) return shipped_shape<64>(p, causal, dtype, v, stream);
    if (D == 128) return shipped_shape<128>(p, causal, dtype, v, stream);
    if (D == 256) return shipped_shape<256>(p, causal, dtype, v, stream);
    return hipErrorInvalidValue;
  }
  if (D == 64) return schedule<V64>(p, causal, dtype, v, stream);
  if (D == 128) return schedule<V128>(p, causal, dtype, v, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
