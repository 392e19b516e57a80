// attn_bwd_kernel.hpp -- gfx950 (CDNA4) kernels of the exact attention
// backward.
//
// Gradients of O = softmax(scale * Q K^T, causal mask) V for a given dO, with
// the probabilities recomputed from the LSE the forward saved (docs.rs page
// "oxicuda-dnn 0.1.8, src/attn/flash_attn/hopper.rs", doc comment of
// FlashAttention3Plan::generate_backward):
//   P_ij = exp(scale q_i.k_j - LSE_i)  (0 where masked)
//   D_i  = rowsum(dO_i * O_i),  dQ = scale dS K      kernel attn_bwd_dq (first)
//   dV = P^T dO, dP = dO V^T, dS = P * (dP - D_i),
//   dK = scale dS^T Q                                kernel attn_bwd_dkdv
// (dS is the gradient of the scaled scores, so the chain rule puts `scale`
// on dK and dQ.)
//
// MI355X mapping:
//   * dK/dV: one workgroup per (key tile, b*H + h); wave w owns 32 keys and
//     keeps their K and V rows in VGPRs as the B operands of S = Q K^T and
//     dP = dO V^T, and their dK^T, dV^T in MFMA accumulators.  Q and dO tiles
//     stream through two LDS stages.  In S and dP (v_mfma_f32_32x32x16) lane
//     l holds key l%32 and 16 query rows in registers, which is exactly the
//     B operand layout of dV^T += dO^T P and dK^T += Q^T dS once packed to 16
//     bits: the A operands dO^T and Q^T come from ds_read_b64_tr_b16.
//   * dQ: one workgroup per (query tile, b*H + h), the forward's shape: Q and
//     dO of 32 queries per wave in VGPRs (B operands of S^T = K Q^T and
//     dP^T = V dO^T: lane l holds query l%32, so LSE_i and D_i are one scalar
//     per lane), K and V tiles stream through LDS, dQ^T += K^T dS^T with K^T
//     read transposed.  This recomputes S and dP once more instead of the
//     page's atomic dQ accumulation: dQ is written once, deterministically.
//     Each wave first forms D_i of its queries from their O and dO rows and
//     writes it out for the dK/dV kernel, which runs second.
//   * The LDS tiles are read both ways (16-byte row reads and transposing
//     reads), so their rows are spread over 1 KiB copy lines in an order that
//     keeps both kinds of read free of bank conflicts (XTile below).
#pragma once

#include "attn_bwd.hpp"
#include "attn_fwd_kernel.hpp"

namespace attn {
namespace bwd {

// LDS tile of ROWS rows of D 16-bit elements, filled by 1 KiB HBM -> LDS copy
// lines (RPL = 512/D rows each) and read two ways:
//   row reads: a 16-lane quarter of a 16-byte read takes the same 16 bytes of
//     16 consecutive rows;
//   transposing reads: 32 lanes take 64 bytes of each of 4 consecutive rows
//     (4 aligned rows 4a..4a+3).
// Line n of a 16-line block holds rows r(n) + 16m (m < RPL) with
// r(n) = 4*(n%4) + n/4, and lines are 1040 bytes apart, so row r (mod 16)
// starts at 16*(4*(r%4) + r/4) modulo the 256-byte bank sweep: 16 consecutive
// rows take 16 distinct 16-byte bank groups, and rows 4a..4a+3 start 64
// bytes apart.  r(n) is its own inverse: row r sits in line r(r).
template <int D_, int ROWS_>
struct XTile {
  static constexpr int D = D_, ROWS = ROWS_;
  static constexpr int ROW_BYTES = 2 * D;
  static constexpr int RPL = 1024 / ROW_BYTES;
  static constexpr int BLOCK_ROWS = 16 * RPL;  // rows of a 16-line block
  static constexpr int LINE = 1024 + 16;
  static constexpr int LINES = ROWS * ROW_BYTES / 1024;
  static constexpr int BYTES = LINES * LINE;
  static constexpr __host__ __device__ int perm(int r16) { return 4 * (r16 % 4) + r16 / 4; }
  static constexpr __host__ __device__ int off(int row) {
    return (row / BLOCK_ROWS) * 16 * LINE + perm(row % 16) * LINE + ((row % BLOCK_ROWS) / 16) * ROW_BYTES;
  }
  // first tile row of copy line n
  static constexpr __host__ __device__ int line_row(int n) { return (n / 16) * BLOCK_ROWS + perm(n % 16); }
  static_assert(ROWS % BLOCK_ROWS == 0, "a tile holds whole 16-line blocks");
};

// The operand addresses below split off(row) into a per-lane part and a
// compile-time part; that is exact when the parts are aligned as checked here.
template <class X>
constexpr bool offsets_split() {
  for (int base = 0; base < X::ROWS; base += 16)
    for (int r = 0; r < 16; ++r)
      if (X::off(base + r) != X::off(base) + X::off(r)) return false;
  for (int base = 0; base < X::ROWS; base += 32)
    for (int r = 0; r < 32; ++r)
      if (X::off(base + r) != X::off(base) + X::off(r)) return false;
  for (int a = 0; a < 16; a += 8)
    for (int r = 0; r < 8; ++r)
      if (X::off(a + r) != X::off(a) + X::off(r)) return false;
  return true;
}

// At D = 256 a wave's operands and accumulators exceed its 256 VGPRs: the
// compiler parks some in AGPRs and, left alone, parks the B-operand
// fragments (K/V rows in dK/dV, Q/dO rows in dQ) there and copies them back
// before their MFMAs (311 moves per 128 MFMAs in dK/dV, 112 per 96 in dQ).
// An MFMA reads its B operand from AGPRs as well, so the fragments are
// pinned there and read in place (bit-identical; backward at B=1 H=8 S=8192
// D=256 causal 929 -> 885 us, B=1 H=16 S=4096 D=256 885 -> 847 us).
// An empty side effect: it keeps a small uniform branch (the mask selects of
// the tiles that need them) a branch, where the compiler would otherwise turn
// it into selects that run on every tile.
__device__ __forceinline__ void keep_branch() { __asm__ volatile(""); }

template <int N>
__device__ __forceinline__ void pin_agprs(u32x4 (&a)[N], u32x4 (&b)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) __asm__ volatile("" : "+a"(a[i]), "+a"(b[i]));
}

// The first row of head bh (= b*H + h) of a tensor with strides s.
template <class T>
__device__ __forceinline__ T* head_ptr(T* base, const Strides& s, uint32_t bh, int H, Div31 dH) {
  const uint32_t b = div31(bh, dH);
  return base + (int64_t)b * s.sb + (int64_t)(bh - b * (uint32_t)H) * s.sh;
}

// HBM -> LDS copies of XTile tiles of one head (rows of D elements, ss
// apart).  Lane i of a copy instruction carries row slot i / (D/8) of the
// line and 16-byte chunk i % (D/8).  Rows at or past `rows` read as 0.
template <class X>
struct XCopier {
  static constexpr int D = X::D;
  const uint16_t* src;
  int rows, ss;
  uint32_t lane_off;
  __device__ __forceinline__ void init(const uint16_t* src_, int ss_, int rows_, int lane) {
    src = src_;
    ss = ss_;
    rows = rows_;
    lane_off = (uint32_t)(16 * (lane / (D / 8)) * ss + (lane % (D / 8)) * 8) * 2u;
  }
  // (the byte count is wave-uniform; readfirstlane keeps it in an SGPR, where
  // a buffer descriptor must be, instead of a loop over distinct lane values)
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile(int r0) const {
    const uint32_t bytes = r0 < rows ? rows_bytes(rows - r0, ss, D) : 0u;
    return make_rsrc(src + (int64_t)r0 * ss, (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes));
  }
  __device__ __forceinline__ void line(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int n) const {
    load16_lds(r, dst + n * X::LINE, lane_off, (uint32_t)(X::line_row(n) * ss) * 2u);
  }
};

// 4 bytes per lane from global memory straight into LDS at lds + 4*lane; a
// lane whose dword lies past the buffer descriptor's end writes 0.
__device__ __forceinline__ void load4_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, (int)byte_off, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc);
template <>
__device__ __forceinline__ float dot2<DT_F16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}
template <>
__device__ __forceinline__ float dot2<DT_BF16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

constexpr float kLog2e = 1.4426950408889634074f;

// Wait for this wave's copies, then for every wave, with scheduling fences on
// both sides: without them the scheduler moves MFMAs of one step across the
// barrier into the next, which keeps two steps' registers live at once.
__device__ __forceinline__ void fenced_sync() {
  __builtin_amdgcn_sched_barrier(0);
  wait_loads();
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Tile shapes per head dim: every tile is one 16-line block of XTile.
template <int D_>
struct BwdCfg {
  static constexpr int D = D_;
  static constexpr int NW = 4;                  // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int STEP = 16 * (512 / D);   // rows of a streamed tile: 128 / 64 / 32
  static constexpr int BN = 32 * NW;            // keys per dK/dV workgroup
  static constexpr int BM = 32 * NW;            // queries per dQ workgroup
  static constexpr int DK = D / 16, DB = D / 32;
  // two waves per SIMD (at most 256 registers each) where the registers
  // allow it: one wave's MFMAs then run beside the other's VALU work
  static constexpr int WAVES_PER_SIMD = D <= 128 ? 2 : 1;
  using X = XTile<D, STEP>;
  static constexpr int LDS_BYTES = 4 * X::BYTES + 4 * 4 * (STEP > 64 ? STEP : 64);  // 2 stages x 2 tiles (+ row values)
  static_assert(offsets_split<X>(), "operand offsets must split into lane and constant parts");
  static_assert(X::LINES % NW == 0, "copy lines must split evenly over the waves");
};

// Store a wave's 32 rows of a [rows, D] output held in the transposed MFMA
// accumulator layout (lane l: row row0 + l%32, columns 32db + 8g + 4*half +
// 0..3), each value times sc and rounded to 16 bits.  Stored directly, one
// store instruction writes 8 bytes into each of 32 rows; STAGED, the wave
// first writes the rows into its own LDS area (padded rows, so the 8-byte
// pieces of 32 rows hit distinct banks), reads them back as whole rows and
// stores 16 contiguous bytes per lane: 8x fewer memory requests at D=128.
template <int D, int DT, bool STAGED>
__device__ __forceinline__ void store_rows(uint8_t* area, const f32x16 (&acc)[D / 32], float sc, uint16_t* head,
                                           int64_t ss, int row0, int rows, int lane) {
  using E = Elem<DT>;
  constexpr int DB = D / 32;
  const int half = lane >> 5, my = row0 + (lane & 31);
  if constexpr (!STAGED) {
    if (my >= rows) return;
    uint16_t* r = head + (int64_t)my * ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = E::pack2(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc);
        w[1] = E::pack2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc);
        *reinterpret_cast<u32x2*>(r + 32 * db + 8 * g + 4 * half) = w;
      }
    }
  } else {
    constexpr int RS = 2 * D + 16;  // staged row stride (bytes)
    uint8_t* mine = area + (lane & 31) * RS;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = E::pack2(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc);
        w[1] = E::pack2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc);
        *reinterpret_cast<u32x2*>(mine + 2 * (32 * db + 8 * g + 4 * half)) = w;
      }
    }
    // a wave's LDS accesses execute in order; keep the compiler from moving
    // the reads above the writes (or a later reuse of the area above them)
    __asm__ volatile("" ::: "memory");
    constexpr int LPR = D / 8, RPI = 64 / LPR;  // lanes per row, rows per store instruction
    const int rl = lane / LPR, cl = lane % LPR;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + rl;
      const u32x4 v = *reinterpret_cast<const u32x4*>(area + r * RS + 16 * cl);
      // whole rows, written once: non-temporal, as the forward's output
      if (row0 + r < rows) store_nt(v, reinterpret_cast<u32x4*>(head + (int64_t)(row0 + r) * ss + 8 * cl));
    }
    __asm__ volatile("" ::: "memory");
  }
}

// Lane part of a transposing read (ds_read_b64_tr_b16) of an XTile: in each
// 16-lane group lane i reads row i/4 of 4 consecutive rows (4*half + i/4
// after the k-slot order of the packed 16-bit operands) at columns
// 4*(i%4)..+3; the second 16-lane group of each half reads 16 columns on.
template <class X>
__device__ __forceinline__ int tr_lane_off(int lane) {
  return X::off(4 * (lane >> 5) + ((lane & 15) >> 2)) + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
}

// A operand (32 rows x 16 head-dim columns) from the transposing reads of
// rows 16*ks + {8r + 4*half + 0..3 : r = 0, 1} at head-dim block db.
template <class X>
__device__ __forceinline__ u32x4 tr_operand(const uint8_t* t, int trl, int ks, int db) {
  const uint8_t* p = t + trl + 64 * db;
  const u32x2 lo = lds_read_tr16(p + X::off(16 * ks));
  const u32x2 hi = lds_read_tr16(p + X::off(16 * ks + 8));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (key tile of BN keys, b*H + h).
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int DT>
__global__ __launch_bounds__(BwdCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(BwdCfg<D>::WAVES_PER_SIMD)))
void attn_bwd_dkdv(const BwdProblem p) {
  using C = BwdCfg<D>;
  using X = typename C::X;
  using E = Elem<DT>;
  constexpr int BQ = C::STEP, MB = BQ / 32, DK = C::DK, DB = C::DB, BN = C::BN;
  constexpr int LPW = X::LINES / C::NW;
  // LSE and D_i of a step's queries go to LDS too, 64 rows per copy
  // instruction (one dword per lane), one instruction per wave
  constexpr int LR = BQ > 64 ? BQ : 64;
  static_assert(2 * (LR / 64) <= C::NW, "one row-value copy per wave");

  __shared__ __attribute__((aligned(1024))) uint8_t qt0[X::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t qt1[X::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ot0[X::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ot1[X::BYTES];
  __shared__ __attribute__((aligned(16))) float ls0[LR];
  __shared__ __attribute__((aligned(16))) float ls1[LR];
  __shared__ __attribute__((aligned(16))) float dl0[LR];
  __shared__ __attribute__((aligned(16))) float dl1[LR];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;

  // key tiles in order of decreasing cost when causal (key tile 0 is seen by
  // the most queries), in chunks of heads per XCD as the forward's query
  // tiles; otherwise contiguous runs per XCD as in the forward
  uint32_t kt, bh32;
  workgroup_tile<CAUSAL>(p.map_k, blockIdx.x, &kt, &bh32);
  const int64_t bh = bh32;
  if (CAUSAL) kt = (uint32_t)p.nk - 1 - kt;
  const int Sq = p.Sq, Skv = p.Skv, koff = Skv - Sq;
  const int k0 = (int)kt * BN, kbase = k0 + 32 * wave, my_k = kbase + col;
  const uint16_t* qh = head_ptr(p.q, p.s_q, bh32, p.H, p.dH);
  const uint16_t* doh = head_ptr(p.dO, p.s_do, bh32, p.H, p.dH);
  const uint16_t* kh = head_ptr(p.k, p.s_k, bh32, p.H, p.dH);
  const uint16_t* vh = head_ptr(p.v, p.s_v, bh32, p.H, p.dH);
  const float* lseh = p.lse + bh * Sq;
  const float* delh = p.delta + bh * Sq;
  const __amdgpu_buffer_rsrc_t lse_r = make_rsrc(lseh, (uint32_t)Sq * 4u);
  const __amdgpu_buffer_rsrc_t del_r = make_rsrc(delh, (uint32_t)Sq * 4u);

  // this wave's keys: B operands of S = Q K^T and dP = dO V^T (rows past Skv read 0)
  u32x4 kf[DK], vf[DK];
  {
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kh, rows_bytes(Skv, p.s_k.ss, D));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vh, rows_bytes(Skv, p.s_v.ss, D));
    const uint32_t koff = (uint32_t)(my_k * p.s_k.ss + 8 * half) * 2u;
    const uint32_t voff = (uint32_t)(my_k * p.s_v.ss + 8 * half) * 2u;
#pragma unroll
    for (int kc = 0; kc < DK; ++kc) {
      kf[kc] = load16(kr, koff + 32 * kc);
      vf[kc] = load16(vr, voff + 32 * kc);
    }
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dka[db] = dva[db] = f32x16{};

  // queries that see any key of the tile: i >= k0 - koff when causal
  int qs = CAUSAL ? k0 - koff : 0;
  qs = qs < 0 ? 0 : qs / BQ * BQ;
  const int n = qs < Sq ? (Sq - qs + BQ - 1) / BQ : 0;

  XCopier<X> qc, oc;
  qc.init(qh, p.s_q.ss, Sq, lane);
  oc.init(doh, p.s_do.ss, Sq, lane);
  auto fetch = [&](int s, uint8_t* dq_, uint8_t* do_, float* ls_, float* dl_) __attribute__((always_inline)) {
    const int r0 = qs + s * BQ;
    const __amdgpu_buffer_rsrc_t rq = qc.tile(r0), ro = oc.tile(r0);
#pragma unroll
    for (int l = 0; l < LPW; ++l) {
      qc.line(rq, dq_, wave * LPW + l);
      oc.line(ro, do_, wave * LPW + l);
    }
    // rows past Sq (or past the step) land as 0 or as unused values
#pragma unroll
    for (int m = 0; m < LR / 64; ++m) {
      const uint32_t off = (uint32_t)(r0 + 64 * m + lane) * 4u;
      if (wave == 2 * m) load4_lds(lse_r, ls_ + 64 * m, off);
      if (wave == 2 * m + 1) load4_lds(del_r, dl_ + 64 * m, off);
    }
  };

  const int xrow = X::off(col) + 16 * half;  // lane part of a row read
  const int trl = tr_lane_off<X>(lane);      // lane part of a transposing read
  const float c = p.c;

  auto step = [&](int s, const uint8_t* qt, const uint8_t* ot, const float* ls, const float* dl)
                  __attribute__((always_inline)) {
    const int q0 = qs + s * BQ;
    // every (query, key) pair of this wave masked, or no key of the wave
    // exists: nothing to add
    if ((CAUSAL && kbase > q0 + BQ - 1 + koff) || kbase >= Skv) return;
    const bool need_mask = CAUSAL && kbase + 31 > q0 + koff;
    // score (query q0 + 32mb + 8g + 4half + t, key my_k) is kept iff
    // 32mb + 8g + t >= my_k - koff - q0 - 4half
    const int lim = my_k - koff - q0 - 4 * half;
    // one 32-query block at a time (S, dP, then P, dS, then dV, dK), fenced,
    // so that only one block's scores and packed operands are live; each MFMA
    // run is a PIPE-deep operand pipeline (operand t+PIPE read from LDS while
    // MFMA t runs), pinned by scheduling groups so that the reads are not all
    // hoisted ahead of the MFMAs
    constexpr int PIPE = 4;
    constexpr int N1 = 2 * DK;      // S and dP MFMAs, alternating
    constexpr int N3 = 2 * 2 * DB;  // dV and dK MFMAs, alternating
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      // dP starts from -D_i of its rows (LDS holds them negated), so the
      // MFMAs leave dP - D_i: one broadcast LDS read per register group gives
      // the 4 rows of that group, in the accumulator's own register order
      if constexpr (C::WAVES_PER_SIMD == 1) pin_agprs(kf, vf);
      f32x16 sa = f32x16{}, dpa;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dl + 32 * mb + 8 * g + 4 * half);
#pragma unroll
        for (int t = 0; t < 4; ++t) dpa[4 * g + t] = d4[t];
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        auto rd = [&](int t) __attribute__((always_inline)) -> u32x4 {
          return *reinterpret_cast<const u32x4*>(((t & 1) ? ot : qt) + xrow + X::off(32 * mb) + 32 * (t >> 1));
        };
        u32x4 buf[PIPE];
#pragma unroll
        for (int t = 0; t < PIPE; ++t) buf[t] = rd(t);
#pragma unroll
        for (int t = 0; t < N1; ++t) {
          const u32x4 a = buf[t % PIPE];
          if (t + PIPE < N1) buf[t % PIPE] = rd(t + PIPE);
          if (t & 1)
            dpa = E::mfma(a, vf[t >> 1], dpa);
          else
            sa = E::mfma(a, kf[t >> 1], sa);
        }
        sched_prologue<0, N1, 0, PIPE>();
        sched_steady<0, N1, 0, PIPE, 0, 1>();
      }
      float pr[16], ds[16];
      // the exp2 offsets of the 4 rows of register group g (one broadcast LDS
      // read per half)
      auto offs = [&](int g) __attribute__((always_inline)) {
        return *reinterpret_cast<const f32x4*>(ls + 32 * mb + 8 * g + 4 * half);
      };
      if constexpr (C::WAVES_PER_SIMD == 2) {
        // the mask selects in a uniform branch of their own (folded into the
        // exp2 loop, they ran on every tile: the compiler merged the tile's
        // need_mask into each select)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = offs(g);
#pragma unroll
          for (int t = 0; t < 4; ++t) pr[4 * g + t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[4 * g + t], c, l4[t]));
        }
        if (need_mask) {
          keep_branch();
#pragma unroll
          for (int i = 0; i < 16; ++i) pr[i] = (32 * mb + 8 * (i >> 2) + (i & 3)) >= lim ? pr[i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = pr[i] * dpa[i];  // P * (dP - D_i)
      } else {
        // D = 256: the select folded in (the form that keeps the operand
        // fragments in place, see pin_agprs; the split form moved them)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = offs(g);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int i = 4 * g + t;
            float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], c, l4[t]));
            if (need_mask) pv = (32 * mb + 8 * g + t) >= lim ? pv : 0.f;
            pr[i] = pv;
            ds[i] = pv * dpa[i];  // P * (dP - D_i)
          }
        }
      }
      u32x4 pf[2], sf[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int b = 8 * s2;
        pf[s2] = u32x4{E::pack2(pr[b], pr[b + 1]), E::pack2(pr[b + 2], pr[b + 3]), E::pack2(pr[b + 4], pr[b + 5]),
                       E::pack2(pr[b + 6], pr[b + 7])};
        sf[s2] = u32x4{E::pack2(ds[b], ds[b + 1]), E::pack2(ds[b + 2], ds[b + 3]), E::pack2(ds[b + 4], ds[b + 5]),
                       E::pack2(ds[b + 6], ds[b + 7])};
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        // op t: s2 = t / (2 DB), db = (t / 2) % DB; even t: dV^T += dO^T P, odd: dK^T += Q^T dS
        auto rd = [&](int t) __attribute__((always_inline)) -> u32x4 {
          return tr_operand<X>((t & 1) ? qt : ot, trl, 2 * mb + t / (2 * DB), (t / 2) % DB);
        };
        u32x4 buf[PIPE];
#pragma unroll
        for (int t = 0; t < PIPE; ++t) buf[t] = rd(t);
#pragma unroll
        for (int t = 0; t < N3; ++t) {
          const u32x4 a = buf[t % PIPE];
          if (t + PIPE < N3) buf[t % PIPE] = rd(t + PIPE);
          const int s2 = t / (2 * DB), db = (t / 2) % DB;
          if (t & 1)
            dka[db] = E::mfma(a, sf[s2], dka[db]);
          else
            dva[db] = E::mfma(a, pf[s2], dva[db]);
        }
        sched_prologue<0, N3, N3, PIPE>();
        sched_steady<0, N3, N3, PIPE, 0, 1>();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // fenced_sync, except that between the wait and the barrier each wave that
  // copied row values turns its rows, just landed, into what the step uses
  // (its own LDS accesses execute in order; the barrier's fence publishes
  // them): the exp2 offsets -LSE * log2(e), one multiply per row instead of
  // one per score, and -D_i, the starting value of dP.  The lane index is
  // recomputed there by an opaque instruction pair: a lane offset hoisted
  // out of the loop would stay live through the MFMA steps, which already
  // take every register.
  auto land = [&](float* ls_, float* dl_) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    wait_loads();
    int ln;
    __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
#pragma unroll
    for (int m = 0; m < LR / 64; ++m) {
      if (wave == 2 * m) ls_[64 * m + ln] = -ls_[64 * m + ln] * kLog2e;
      if (wave == 2 * m + 1) dl_[64 * m + ln] = -dl_[64 * m + ln];
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  if (n > 0) fetch(0, qt0, ot0, ls0, dl0);
  for (int s = 0; s < n; s += 2) {
    land(ls0, dl0);
    if (s + 1 < n) fetch(s + 1, qt1, ot1, ls1, dl1);
    step(s, qt0, ot0, ls0, dl0);
    if (s + 1 >= n) break;
    land(ls1, dl1);
    if (s + 2 < n) fetch(s + 2, qt0, ot0, ls0, dl0);
    step(s + 1, qt1, ot1, ls1, dl1);
  }

  // dK, dV: through LDS where a wave's 32 padded rows fit in one stage array
  // (D <= 128; every wave is done with the stages after this barrier, and
  // no copy is in flight), except in the causal D=128 kernel, whose loop
  // takes all 256 registers: there the staging code made the compiler spill
  constexpr bool STAGED = 32 * (2 * D + 16) <= X::BYTES && !(CAUSAL && D == 128);
  if constexpr (STAGED) __syncthreads();
  uint8_t* const area = wave == 0 ? qt0 : wave == 1 ? qt1 : wave == 2 ? ot0 : ot1;
  store_rows<D, DT, STAGED>(area, dka, p.scale, head_ptr(p.dk, p.s_dk, bh32, p.H, p.dH), p.s_dk.ss, kbase, Skv, lane);
  store_rows<D, DT, STAGED>(area, dva, 1.f, head_ptr(p.dv, p.s_dv, bh32, p.H, p.dH), p.s_dv.ss, kbase, Skv, lane);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (query tile of BM queries, b*H + h).
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int DT>
__global__ __launch_bounds__(BwdCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(BwdCfg<D>::WAVES_PER_SIMD)))
void attn_bwd_dq(const BwdProblem p) {
  using C = BwdCfg<D>;
  using X = typename C::X;
  using E = Elem<DT>;
  constexpr int BNK = C::STEP, NB = BNK / 32, DK = C::DK, DB = C::DB, BM = C::BM;
  constexpr int LPW = X::LINES / C::NW;

  __shared__ __attribute__((aligned(1024))) uint8_t kt0[X::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kt1[X::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vt0[X::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vt1[X::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;

  uint32_t tile, bh32;
  workgroup_tile<CAUSAL>(p.map_q, blockIdx.x, &tile, &bh32);
  const int64_t bh = bh32;
  const int Sq = p.Sq, Skv = p.Skv, koff = Skv - Sq;
  const int q0 = (int)tile * BM, wq_first = q0 + 32 * wave, my_q = wq_first + col;
  const uint16_t* kh = head_ptr(p.k, p.s_k, bh32, p.H, p.dH);
  const uint16_t* vh = head_ptr(p.v, p.s_v, bh32, p.H, p.dH);

  // this wave's queries: B operands of S^T = K Q^T and dP^T = V dO^T (lane
  // l: query l%32, columns 16kc + 8half + 0..7; rows past Sq read 0)
  u32x4 qf[DK], of[DK];
  float dl;  // D_i = rowsum(dO_i * O_i), fp32
  {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(head_ptr(p.q, p.s_q, bh32, p.H, p.dH), rows_bytes(Sq, p.s_q.ss, D));
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(head_ptr(p.dO, p.s_do, bh32, p.H, p.dH), rows_bytes(Sq, p.s_do.ss, D));
    const __amdgpu_buffer_rsrc_t our = make_rsrc(head_ptr(p.o, p.s_o, bh32, p.H, p.dH), rows_bytes(Sq, p.s_o.ss, D));
    const uint32_t qoff = (uint32_t)(my_q * p.s_q.ss + 8 * half) * 2u;
    const uint32_t ooff = (uint32_t)(my_q * p.s_do.ss + 8 * half) * 2u;
    const uint32_t uoff = (uint32_t)(my_q * p.s_o.ss + 8 * half) * 2u;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < DK; ++kc) {
      qf[kc] = load16(qr, qoff + 32 * kc);
      of[kc] = load16(orr, ooff + 32 * kc);
      const u32x4 ov = load16(our, uoff + 32 * kc);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = dot2<DT>(ov[e], of[kc][e], acc[e]);
    }
    // this lane's half of the row, plus the other half's (lane l ^ 32)
    dl = sum_halves((acc[0] + acc[1]) + (acc[2] + acc[3]));
  }
  const bool q_ok = my_q < Sq;
  const float nl = q_ok ? -p.lse[bh * Sq + my_q] * kLog2e : 0.f;
  if (q_ok && half == 0) p.delta[bh * Sq + my_q] = dl;
  f32x16 dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = f32x16{};
  // -D_i in every entry: the accumulator operand of each block's first dP
  // MFMA, so the MFMAs leave dP - D_i (as in the dK/dV kernel) and no
  // subtraction runs per score (16 VALU instructions per 32-key block)
  f32x16 negd;
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = -dl;

  const int q_end = q0 + BM < Sq ? q0 + BM : Sq;
  int kv_end = CAUSAL ? q_end + koff : Skv;
  kv_end = kv_end < Skv ? kv_end : Skv;
  const int n = kv_end > 0 ? (kv_end + BNK - 1) / BNK : 0;

  XCopier<X> kc_, vc_;
  kc_.init(kh, p.s_k.ss, Skv, lane);
  vc_.init(vh, p.s_v.ss, Skv, lane);
  auto fetch = [&](int j, uint8_t* k_, uint8_t* v_) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rk = kc_.tile(j * BNK), rv = vc_.tile(j * BNK);
#pragma unroll
    for (int l = 0; l < LPW; ++l) {
      kc_.line(rk, k_, wave * LPW + l);
      vc_.line(rv, v_, wave * LPW + l);
    }
  };

  const int xrow = X::off(col) + 16 * half;
  const int trl = tr_lane_off<X>(lane);
  const float c = p.c;
  const int last = CAUSAL ? (my_q + koff < Skv - 1 ? my_q + koff : Skv - 1) : Skv - 1;

  auto step = [&](int j, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
    const int kv0 = j * BNK;
    if (wq_first >= Sq || (CAUSAL && kv0 > wq_first + 31 + koff)) return;
    const bool need_mask = (kv0 + BNK > Skv) || (CAUSAL && kv0 + BNK - 1 > wq_first + koff);
    // score (key kv0 + 32kb + 8g + 4half + t, query my_q) kept iff key <= last
    const int lim = last - kv0 - 4 * half;
    // one 32-key block at a time, each MFMA run a pinned PIPE-deep operand
    // pipeline (as in the dK/dV kernel); the masking code only in the
    // (uniform) branch of the tiles that need it
    constexpr int PIPE = 4;
    constexpr int N1 = 2 * DK;  // S^T and dP^T MFMAs, alternating
    constexpr int N3 = 2 * DB;  // dQ^T MFMAs
    auto blocks = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        if constexpr (C::WAVES_PER_SIMD == 1) pin_agprs(qf, of);
        f32x16 sa = f32x16{}, dpa;
        {
          auto rd = [&](int t) __attribute__((always_inline)) -> u32x4 {
            return *reinterpret_cast<const u32x4*>(((t & 1) ? vt : kt) + xrow + X::off(32 * kb) + 32 * (t >> 1));
          };
          u32x4 buf[PIPE];
#pragma unroll
          for (int t = 0; t < PIPE; ++t) buf[t] = rd(t);
#pragma unroll
          for (int t = 0; t < N1; ++t) {
            const u32x4 a = buf[t % PIPE];
            if (t + PIPE < N1) buf[t % PIPE] = rd(t + PIPE);
            if (t & 1)
              dpa = E::mfma(a, of[t >> 1], t == 1 ? negd : dpa);
            else
              sa = E::mfma(a, qf[t >> 1], sa);
          }
          sched_prologue<0, N1, 0, PIPE>();
          sched_steady<0, N1, 0, PIPE, 0, 1>();
        }
        // the mask selects run in a uniform branch of their own: with two
        // copies of the whole block (masked and not) the compiler gave the
        // dQ^T accumulators different registers in each and copied all of
        // them at every step (64 moves at D=128)
        float pv[16], ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], c, nl));
        if (need_mask) {
          keep_branch();
#pragma unroll
          for (int i = 0; i < 16; ++i) pv[i] = (32 * kb + 8 * (i >> 2) + (i & 3)) <= lim ? pv[i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = pv[i] * dpa[i];  // P * (dP - D_i)
        u32x4 sf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int b = 8 * s2;
          sf[s2] = u32x4{E::pack2(ds[b], ds[b + 1]), E::pack2(ds[b + 2], ds[b + 3]), E::pack2(ds[b + 4], ds[b + 5]),
                         E::pack2(ds[b + 6], ds[b + 7])};
        }
        __builtin_amdgcn_sched_barrier(0);
        {
          // op t: s2 = t / DB, db = t % DB
          auto rd = [&](int t) __attribute__((always_inline)) -> u32x4 {
            return tr_operand<X>(kt, trl, 2 * kb + t / DB, t % DB);
          };
          u32x4 buf[PIPE];
#pragma unroll
          for (int t = 0; t < PIPE; ++t) buf[t] = rd(t);
#pragma unroll
          for (int t = 0; t < N3; ++t) {
            const u32x4 a = buf[t % PIPE];
            if (t + PIPE < N3) buf[t % PIPE] = rd(t + PIPE);
            dqa[t % DB] = E::mfma(a, sf[t / DB], dqa[t % DB]);
          }
          sched_prologue<0, N3, N3, PIPE>();
          sched_steady<0, N3, N3, PIPE, 0, 1>();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    blocks();
  };

  if (n > 0) fetch(0, kt0, vt0);
  for (int j = 0; j < n; j += 2) {
    fenced_sync();
    if (j + 1 < n) fetch(j + 1, kt1, vt1);
    step(j, kt0, vt0);
    if (j + 1 >= n) break;
    fenced_sync();
    if (j + 2 < n) fetch(j + 2, kt0, vt0);
    step(j + 1, kt1, vt1);
  }

  // dQ: through LDS where a wave's 32 padded rows fit in one stage array
  constexpr bool STAGED = 32 * (2 * D + 16) <= X::BYTES;
  if constexpr (STAGED) __syncthreads();
  uint8_t* const area = wave == 0 ? kt0 : wave == 1 ? kt1 : wave == 2 ? vt0 : vt1;
  store_rows<D, DT, STAGED>(area, dqa, p.scale, head_ptr(p.dq, p.s_dq, bh32, p.H, p.dH), p.s_dq.ss, wq_first, Sq, lane);
}

}  // namespace bwd
}  // namespace attn
