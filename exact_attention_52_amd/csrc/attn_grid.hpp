// attn_grid.hpp -- the workgroup -> (query or key tile, b*H + h) map of the
// forward and backward kernels, and the integer divisions it needs, with every
// divisor fixed on the host before the launch.
//
// A workgroup computes its tile and head before its first load, and an
// integer division by a value known only at run time is a sequence of ~40
// instructions per quotient (a 64-bit one several times that); the map and
// the batch/head split took ~3000 cycles per workgroup that way (timestamp
// probe, B=16 H=32 S=1024 D=64 causal), while its first copies waited.
// With the divisors turned into multipliers on the host each quotient is a
// multiply-high and a shift.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// n / d for a divisor d fixed at launch and every n < 2^31: with
// l = ceil(log2 d), m = ceil(2^(31+l) / d) and s = 31 + l, n / d equals
// (n * m) >> s (Granlund and Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994, theorem 4.2 with N = 31: m * d exceeds
// 2^(31+l) by less than d <= 2^l).  m < 2^32 because d > 2^(l-1).
struct Div31 {
  uint32_t m, s;
};

__host__ __device__ inline Div31 make_div31(uint32_t d) {
  if (d == 0) d = 1;  // never divided by; keeps the multiplier defined
  uint32_t l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  const uint64_t p = (uint64_t)1 << (31 + l);
  return Div31{(uint32_t)((p + d - 1) / d), 31 + l};
}

__host__ __device__ __forceinline__ uint32_t div31(uint32_t n, Div31 v) {
  return (uint32_t)(((uint64_t)n * v.m) >> v.s);
}

// Heads per chunk of the causal order below: as many as keep the chunk's K
// and V rows within kL2ChunkBytes of the XCD's L2.
constexpr int64_t kL2ChunkBytes = (int64_t)4 << 20;
__host__ __device__ inline int64_t causal_head_chunk(int64_t Skv, int64_t D) {
  const int64_t kv = 4 * Skv * D;  // K and V rows of one head, 16-bit
  const int64_t c = kv > 0 ? kL2ChunkBytes / kv : kL2ChunkBytes;
  return c > 1 ? c : 1;
}

// Workgroup id -> (query tile, b*H + h).  Workgroups are handed to the 8 XCDs
// round-robin in id order, so id g runs on XCD g % 8, and each XCD gives its
// next workgroup to the first CU that frees up.
//   Causal: tile costs differ (query tile t has t+1 tiles' worth of keys), so
//   each XCD runs its tiles longest first (list scheduling in
//   longest-processing-time order pairs long and short tiles on each CU).
//   When heads is a multiple of 8, head h runs on XCD h % 8, and each XCD
//   works through its heads `hchunk` at a time: all tiles of a chunk of heads
//   in order of decreasing cost, then the next chunk.  The K/V rows the
//   XCD's running workgroups read then belong to a few heads and stay in its
//   4 MB L2 (with every head's last tile first, 64 heads' K/V at once went
//   through HBM 3.15x over).  hchunk >= heads / 8 gives one chunk: plain
//   longest-first over the XCD's heads.  Otherwise (heads not a multiple of
//   8) id g takes the (g / heads)-th tile counted from the last and head
//   g % heads.
//   Non-causal: equal costs; each XCD gets a contiguous run of logical work
//   (whole heads where the counts allow), in head order.
// The backward's kernels use the same map over key tiles (dK/dV) and query
// tiles (dQ).  Grids stay below 2^31 workgroups (checked before a launch),
// so every quotient below has a numerator < 2^31.
struct TileMap {
  uint32_t nq;         // tiles per head
  uint32_t base, rem;  // non-causal: G / 8, G % 8
  uint32_t chunked;    // causal: 1 for the per-XCD chunks of heads, 0 for longest first over the grid
  uint32_t heads;      // causal: G / nq
  uint32_t hx, c, cnq, clast;  // chunked: heads per XCD, heads per chunk, c * nq, heads of a short last chunk
  Div31 d_nq, d_heads, d_cnq, d_c, d_clast;
};

// G workgroups over nq tiles per head; hchunk as from causal_head_chunk.
__host__ __device__ inline TileMap make_tile_map(int64_t G, int64_t nq, bool causal, int64_t hchunk) {
  constexpr uint32_t X = 8;
  TileMap m = {};
  m.nq = (uint32_t)nq;
  m.d_nq = make_div31(m.nq);
  m.base = (uint32_t)(G / X);
  m.rem = (uint32_t)(G % X);
  m.heads = nq > 0 ? (uint32_t)(G / nq) : 0;
  m.d_heads = make_div31(m.heads);
  const uint32_t hc = hchunk > (int64_t)m.heads ? m.heads : (uint32_t)(hchunk > 0 ? hchunk : 0);
  m.chunked = causal && m.heads % X == 0 && hc > 0;
  m.hx = m.heads / X;
  m.c = hc < m.hx ? hc : m.hx;
  m.cnq = m.c * m.nq;
  m.clast = m.c > 0 ? m.hx % m.c : 0;
  m.d_cnq = make_div31(m.cnq);
  m.d_c = make_div31(m.c);
  m.d_clast = m.clast > 0 ? make_div31(m.clast) : m.d_c;
  return m;
}

template <bool CAUSAL>
__host__ __device__ __forceinline__ void workgroup_tile(const TileMap& m, uint32_t g, uint32_t* tile, uint32_t* bh) {
  constexpr uint32_t X = 8;
  const uint32_t xcd = g % X, slot = g / X;
  if constexpr (CAUSAL) {
    if (!m.chunked) {
      const uint32_t t = div31(g, m.d_heads);
      *bh = g - t * m.heads;
      *tile = m.nq - 1 - t;
      return;
    }
    const uint32_t chunk = div31(slot, m.d_cnq);
    const uint32_t r = slot - chunk * m.cnq;
    const bool short_last = m.hx - chunk * m.c < m.c;  // the last chunk holds hx % c heads
    const uint32_t cw = short_last ? m.clast : m.c;  // heads in this chunk
    const uint32_t t = div31(r, short_last ? m.d_clast : m.d_c);
    *tile = m.nq - 1 - t;
    *bh = (chunk * m.c + (r - t * cw)) * X + xcd;
  } else {
    const uint32_t logical = xcd * m.base + (xcd < m.rem ? xcd : m.rem) + slot;
    const uint32_t b = div31(logical, m.d_nq);
    *bh = b;
    *tile = logical - b * m.nq;
  }
}

}  // namespace attn
