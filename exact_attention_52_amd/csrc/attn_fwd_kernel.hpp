// attn_fwd_kernel.hpp -- gfx950 (CDNA4) kernels of the exact attention forward.
//
// Computes, per (batch*head, query tile), O = softmax(scale * Q K^T, causal
// mask) V and LSE with an online softmax: a running max m and running sum l
// per query row, the partial output rescaled when m grows, and the final
// O = O_acc / l, LSE = m + log l (docs.rs page "oxicuda-dnn 0.1.8,
// src/attn/flash_attn/hopper.rs", doc comment of
// FlashAttention3Plan::generate_forward).
//
// MI355X mapping (differs from the page's Hopper design on purpose):
//   * One workgroup per (query tile of BM = 32*QW rows, b*H + h).  QW*KW waves
//     of 64 lanes: wave (qw, kw) owns 32 query rows and the kw-th 1/KW slice
//     of every key tile.  The Q fragment of a wave lives in VGPRs for the
//     whole kernel; O and (m, l) live in VGPRs (the page keeps them in shared
//     memory).
//   * The score block is computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{f16,bf16}: lane l then holds 16 scores of the
//     single query column l%32 per 32-key block, so the row max/sum is an
//     in-register reduction plus one exchange between lane l and l^32, and
//     the rescale of O^T by exp2(m_old - m_new) is one scalar per lane.
//   * The probabilities, packed to 16 bits, are already the B operand of the
//     second contraction O^T += V^T P^T: no LDS round trip for P.  V stays
//     row-major in LDS and its transposed A operand is read with gfx950's
//     ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x 16-d block and
//     gets it back one d column per lane); the 4-key row groups are picked to
//     match the key order of the packed P registers.
//   * K and V tiles stream through two or three LDS stages, copied straight
//     from HBM into LDS by 16-byte buffer loads while earlier tiles are
//     computed.  Row strides are padded so the 16-byte K reads (8 rows per
//     bank sweep) and the transposing V reads (4 rows of 32 bytes) hit
//     disjoint banks.
//   * exp2/log2 are the hardware v_exp_f32/v_log_f32 with the scale folded
//     as c = scale*log2(e); P and O are rounded to nearest-even.
//   * Causal: key tiles wholly after a wave's last query are skipped (or, in
//     the kernels that pipeline across waves or tiles, get P = 0), and only
//     tiles crossing the diagonal (or the ragged end) are masked.
//   * Three schedules of the same per-wave steps: kernel 1 (each wave runs
//     qk, softmax, pv per tile; several workgroups per CU at D=64), kernel 2
//     (D=128: two wave groups per SIMD alternate MFMA and softmax phases) and
//     kernel 3 (D=256 on large grids: one wave per SIMD interleaves the next
//     tile's qk and the previous tile's pv MFMAs with this tile's softmax).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "attn_grid.hpp"

namespace attn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };

// ---------------------------------------------------------------------------
// Element-type helpers
// ---------------------------------------------------------------------------
template <int DT>
struct Elem;

template <>
struct Elem<DT_F16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // x rounded to the nearest-even 16-bit value, back in fp32
  static __device__ __forceinline__ float round(float x) { return (float)(_Float16)x; }
  // Two fp32 values -> packed 16-bit pair, round to nearest even.
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
};

template <>
struct Elem<DT_BF16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float round(float x) { return (float)(__bf16)x; }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
};

// ---------------------------------------------------------------------------
// Tile configuration and LDS layout
// ---------------------------------------------------------------------------
// K and V tiles are copied HBM -> LDS by buffer_load_dwordx4 ... lds, where
// one wave instruction writes 1 KiB: lane i's 16 bytes land at base + 16*i.
// Each such 1 KiB "line" holds RPL = 512/D whole rows of the tile, and lines
// are padded so that the operand reads hit distinct banks of the 64 x 4-byte
// LDS (256 bytes per bank sweep):
//   K: line L of a 16-line block holds rows L, L+16, L+32, ... (pad 16 B), so
//      the 16 consecutive rows read by one 16-lane quarter of a 16-byte
//      operand read sit 16 bytes apart modulo 256; a tile of fewer lines
//      (8 at D=64 with 64 keys) forms one block of all its lines, rows L,
//      L+8, ..., and the 8 rows that one 128-byte read cycle serves still
//      fall in distinct 16-byte slots;
//   V: line L of a 4-line block holds rows L, L+4, ... (pad 64 B), so the 4
//      consecutive rows of a transposing read, 64 bytes wide across two
//      16-lane groups, sit 64 bytes apart modulo 256.
template <int D_, int QW_, int KW_, int BN_, bool PINGPONG_ = false, bool STAGGER_ = false, int STAGES_ = 2,
          bool PRODUCER_ = false, bool INWAVE_ = false>
struct TileCfg {
  static constexpr bool PINGPONG = PINGPONG_;  // use the two-group ping-pong kernel
  static constexpr bool INWAVE = INWAVE_;      // use the in-wave pipelined kernel (kernel 3)
  static constexpr bool STAGGER = STAGGER_;    // kernel 1: staggered K/V copies, two barriers per tile
  // kernel 1 without STAGGER: LDS stages of K/V (1, 2 or 3), and whether one
  // extra wave issues every HBM -> LDS copy while the others only compute
  static constexpr int STAGES = STAGES_;
  static constexpr bool PRODUCER = PRODUCER_;
  static constexpr int D = D_;
  static constexpr int QW = QW_;             // waves along query rows
  static constexpr int KW = KW_;             // waves along each key tile
  static constexpr int BN = BN_;             // keys per tile
  static constexpr int BM = 32 * QW;         // query rows per workgroup
  static constexpr int NW = QW * KW;         // computing waves per workgroup
  static constexpr int NT = 64 * (NW + (PRODUCER ? 1 : 0));  // threads per workgroup
  static constexpr int KSUB = BN / KW;       // keys per wave per tile
  static constexpr int NB = KSUB / 32;       // 32-key blocks per wave per tile
  static constexpr int DK = D / 16;          // k-steps of the score MFMA
  static constexpr int DB = D / 32;          // 32-row blocks of O^T
  static constexpr int ROW_BYTES = 2 * D;
  static constexpr int RPL = 1024 / ROW_BYTES;           // rows per 1 KiB line
  static constexpr int LINES = BN * ROW_BYTES / 1024;    // lines per tile
  static constexpr int K_LINE = 1024 + 16;
  static constexpr int V_LINE = 1024 + 64;
  static constexpr int K_TILE = LINES * K_LINE;
  static constexpr int V_TILE = LINES * V_LINE;
  static constexpr int KV_LDS_BYTES = STAGES * (K_TILE + V_TILE);
  static constexpr int LOADS_PER_WAVE = LINES / NW;      // K lines (and V lines) per wave
  // plus, with a key split, the per-row l, m, p_top and e_top of the merged
  // partials
  static constexpr int LDS_BYTES = KV_LDS_BYTES + (KW > 1 ? (KW - 1) * QW * 4 * 64 * 4 : 0);

  // K lines form blocks of KB lines (16, or all the lines of a smaller
  // tile); line L of a block holds rows L, L + KB, ...
  static constexpr int KB = LINES < 16 ? LINES : 16;
  // byte offset of tile row `row` inside a K / V tile
  static constexpr __host__ __device__ int k_off(int row) {
    return (row / (KB * RPL)) * KB * K_LINE + (row % KB) * K_LINE + ((row % (KB * RPL)) / KB) * ROW_BYTES;
  }
  static constexpr __host__ __device__ int v_off(int row) {
    return (row / (4 * RPL)) * 4 * V_LINE + (row % 4) * V_LINE + ((row % (4 * RPL)) / 4) * ROW_BYTES;
  }
  // first tile row of load line n (the line's rows step by 16 for K, 4 for V)
  static constexpr __host__ __device__ int k_line_row(int n) { return (n / KB) * KB * RPL + n % KB; }
  static constexpr __host__ __device__ int v_line_row(int n) { return (n / 4) * 4 * RPL + n % 4; }

  static_assert(D % 32 == 0 && RPL >= 1, "head dim must be a multiple of 32, at most 512");
  static_assert(KSUB % 32 == 0 && NB >= 1, "each wave needs whole 32-key blocks");
  static_assert(BN % (KB * RPL) == 0 && KB >= 8, "tile must hold whole K line blocks of >= 8 lines");
  static_assert(LINES % NW == 0, "load lines must split evenly over the waves");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
  static_assert(STAGES >= 1 && STAGES <= 3, "1 to 3 K/V stages");
  static_assert(STAGES == 2 || (!PINGPONG && !STAGGER), "the ping-pong and staggered schedules use 2 stages");
  static_assert(!PRODUCER || (!PINGPONG && !STAGGER && KW == 1), "a producer wave only in kernel 1, KW = 1");
  static_assert(!INWAVE || (!PINGPONG && !STAGGER && !PRODUCER && STAGES == 2), "the in-wave pipeline: two stages");
};

typedef short s16x4 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// ds_read_b64_tr_b16: within each 16-lane group, lane i supplies the address
// of 4 consecutive 16-bit elements of row i/4 (columns 4*(i%4)..+3) of a
// 4 x 16 block and receives column i of the block's 4 rows.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Lane l and lane l^32 combined, in every lane (v_permlane32_swap returns
// both halves' values without a trip through LDS).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)r[0]),
                                      __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Maximum of x[0..N-1] as a tree of 3-input maxima (v_maximum3_f32: IEEE
// maximum, no canonicalising moves; the inputs are never NaN): N/2 steps.
template <int N>
__device__ __forceinline__ float max_tree(const float* x) {
  if constexpr (N == 1) {
    return x[0];
  } else if constexpr (N == 2) {
    return __builtin_elementwise_maximum(x[0], x[1]);
  } else {
    constexpr int M = N / 3 + (N % 3 != 0);
    float y[M];
#pragma unroll
    for (int i = 0; i < N / 3; ++i)
      y[i] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[3 * i], x[3 * i + 1]), x[3 * i + 2]);
    if constexpr (N % 3 == 1) y[N / 3] = x[N - 1];
    if constexpr (N % 3 == 2) y[N / 3] = __builtin_elementwise_maximum(x[N - 2], x[N - 1]);
    return max_tree<M>(y);
  }
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, in order
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Keep the computation of x where it is written: the empty volatile asm uses
// x, so the value must exist at this point (the compiler would otherwise sink
// work whose results are only read later, e.g. P computed for the next
// tile's MFMAs, out of the slot it was placed in).
template <class T>
__device__ __forceinline__ void pin(const T& x) {
  __asm__ volatile("" ::"v"(x));
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmem = 0x010;
constexpr int kSchedDsRead = 0x100;

// LDS read instructions of pipeline operand T: 2 transposing reads for a PV
// operand (T < NPV), 1 for a score operand, none past the end.
template <int T, int NOPS, int NPV>
constexpr int op_reads() {
  return T < NOPS ? (T < NPV ? 2 : 1) : 0;
}

// Does MFMA T of a block carry one of NL copy instructions (one after every
// LSTRIDE-th MFMA, from the first)?
template <int T, int NL, int LSTRIDE>
constexpr bool copy_after() {
  return NL > 0 && T % LSTRIDE == 0 && T / LSTRIDE < NL;
}

// Scheduling groups for a PIPE-deep operand pipeline of NOPS MFMAs: the
// reads of operands 0..PIPE-1, then for each T: MFMA T, reads of T+PIPE, and
// the copy instruction that goes with MFMA T, if any.
template <int T, int NOPS, int NPV, int PIPE>
__device__ __forceinline__ void sched_prologue() {
  if constexpr (T < PIPE) {
    if constexpr (op_reads<T, NOPS, NPV>() > 0)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, op_reads<T, NOPS, NPV>(), 0);
    sched_prologue<T + 1, NOPS, NPV, PIPE>();
  }
}
template <int T, int NOPS, int NPV, int PIPE, int NL, int LSTRIDE>
__device__ __forceinline__ void sched_steady() {
  if constexpr (T < NOPS) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (op_reads<T + PIPE, NOPS, NPV>() > 0)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, op_reads<T + PIPE, NOPS, NPV>(), 0);
    if constexpr (copy_after<T, NL, LSTRIDE>()) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
    sched_steady<T + 1, NOPS, NPV, PIPE, NL, LSTRIDE>();
  }
}

// Copy hook of an MFMA block that issues no copies.
struct NoCopy {
  __device__ __forceinline__ void operator()(int) const {}
};

// Buffer descriptor over `bytes` bytes at `base`: loads past the end return
// zero, which pads the ragged last tile without any select after the load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}

// The staged epilogue writes O as whole rows, once: those stores carry the
// non-temporal hint.  Measured (one process, A/B, with the LSE stores hinted
// too): B=4 H=16 S=2048 D=128 causal bf16 75.7 -> 73.8 us, B=16 H=32 S=1024
// D=64 causal bf16 99.0 -> 97.1 us, the fp16 D=64 case level.  The same hint
// on the Q loads cut the HBM bytes read (by 7 % and 13 %) but made both
// cases slower, and on the backward's stores it cost the kernels that write
// 8-byte pieces of rows up to 27 %; so partial-row stores stay unhinted.
template <class T>
__device__ __forceinline__ void store_nt(T v, T* p) {
  __builtin_nontemporal_store(v, p);
}

// 16 bytes per lane from global memory straight into LDS at lds + 16*lane;
// the source is byte_off (per lane) + wave_off (wave-uniform, an SGPR).  On
// gfx950 the buffer range check covers the sum of both: a lane whose 16 bytes
// lie past the descriptor's end writes zeros (measured with a NaN-filled tail
// past the tensor), so the wave-uniform row offset can stay in a scalar.
__device__ __forceinline__ void load16_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t byte_off,
                                           uint32_t wave_off = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, (int)byte_off, (int)wave_off, 0, 0);
}

// Running-max hysteresis (log2 units): O, l are only rescaled when some row's
// max grows by more than this; otherwise P is taken against the old max and
// may reach 2^8, which fp16/bf16 P and fp32 sums hold with unchanged
// relative precision.
constexpr float kRescaleSlack = 8.0f;


// ---------------------------------------------------------------------------
// The problem in global memory
// ---------------------------------------------------------------------------
// Q, O [B,H,Sq,D] and K, V [B,H,Skv,D] of 16-bit elements, each row of D
// elements contiguous and addressed by batch, head and row strides (in
// elements); LSE [B,H,Sq] contiguous fp32.  Causal keeps key j for query i iff
// j <= i + (Skv - Sq): the last query sees the last key.
struct Problem {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;  // batch, head strides
  int q_ss, k_ss, v_ss, o_ss;                              // row strides (>= D)
  int Sq, Skv, H, nq;                                      // nq query tiles per head
  int64_t G;                                               // workgroups
  int64_t hchunk;                                          // heads per chunk (causal order)
  TileMap map;                                             // workgroup -> (query tile, b*H + h)
  Div31 dH;                                                // division by H
  float c;                                                 // |scale| * log2(e), > 0
  uint32_t qsign;  // 0x80008000 when scale < 0: Q is negated in registers
};

// One (b, h) of the problem.
struct HeadView {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int q_ss, k_ss, v_ss, o_ss;
  int Sq, Skv, koff;  // koff = Skv - Sq
  uint32_t qsign;     // XOR mask of every 32-bit word of the Q fragment
};

__device__ __forceinline__ HeadView head_view(const Problem& p, uint32_t bh) {
  const uint32_t b32 = div31(bh, p.dH);
  const int64_t b = b32, h = bh - b32 * (uint32_t)p.H;
  HeadView hv;
  hv.q = p.q + b * p.q_sb + h * p.q_sh;
  hv.k = p.k + b * p.k_sb + h * p.k_sh;
  hv.v = p.v + b * p.v_sb + h * p.v_sh;
  hv.o = p.o + b * p.o_sb + h * p.o_sh;
  hv.lse = p.lse + (int64_t)bh * p.Sq;
  hv.q_ss = p.q_ss, hv.k_ss = p.k_ss, hv.v_ss = p.v_ss, hv.o_ss = p.o_ss;
  hv.Sq = p.Sq, hv.Skv = p.Skv, hv.koff = p.Skv - p.Sq;
  hv.qsign = p.qsign;
  return hv;
}

// Bytes spanned by n rows of D 16-bit elements at row stride ss (0 if none):
// a buffer descriptor of this size returns 0 for every row >= n.
__device__ __forceinline__ uint32_t rows_bytes(int n, int ss, int D) {
  return n > 0 ? (uint32_t)((n - 1) * ss + D) * 2u : 0u;
}

// ---------------------------------------------------------------------------
// Per-wave state and the three steps of one key tile
// ---------------------------------------------------------------------------
// A wave owns 32 query rows (one per lane column) and the kw-th slice of
// every key tile.  Per tile j it runs
//   qk(j)      S^T = K_j Q^T into sacc (MFMA),
//   softmax(j) mask, running max, rescale factor, P = exp2(c*s - m) packed
//              into pf, row sums (VALU),
//   pv(j)      O^T += V_j^T P^T (MFMA),
// in that order; the kernels below only decide how these steps of different
// waves and tiles are interleaved.
template <class C, bool CAUSAL, int DT>
struct Wave {
  using E = Elem<DT>;
  static constexpr int D = C::D, BN = C::BN, NB = C::NB, DK = C::DK, DB = C::DB;

  u32x4 qf[DK];      // Q fragment (B operand of S^T), resident
  f32x16 oacc[DB];   // O^T accumulator
  f32x16 sacc[NB];   // scores of the tile between qk and softmax
  u32x4 pf[2 * NB];  // packed P of the tile between softmax and pv
  float m_run;       // reference max of c*s (log2 units), lagging the true
                     // running max by less than kRescaleSlack
  float nm_ref;      // -m_run, or 0 while m_run is -inf: the exp2 offset
  float m_thr;       // m_run + kRescaleSlack: scores above it force a rescale
  float l_run;       // partial running sum of the fp32 P over this lane's keys
  float p_top;       // the row's largest P so far (fp32) ...
  float e_top;       // ... and round16(P) - P for it.  O is normalised by
                     // (sum of P) + e_top: the dominant key's weight is then
                     // the same rounded P the MFMA used (to first order the
                     // error is sum over the other keys j of w_j d_j V_j, d_j
                     // their relative rounding), while the plain fp32 sum
                     // would add w* d* V* of the dominant key: 2.03e-3 on a
                     // peaky fp16 row with |O| ~ 4.5, over the 2e-3 bound
  bool pend_rs;      // the last deferred softmax asked for a rescale of O^T
                     // (wave-uniform: the caller skips the multiplies when not)
  float alpha;       // exp2(old m_run - new m_run) of the last softmax: the
                     // factor O^T still owes when the rescale is deferred
  int lane, half, wq_first, wq_last, my_q, kbase, Sq, Skv, koff, k_lane, v_lane;
  float c;
  uint32_t qsign;  // a negative scale is applied as -Q (exact) times |scale|

  // LOAD_Q = false leaves qf to copy_q / read_q below
  template <bool LOAD_Q = true>
  __device__ __forceinline__ void init(const HeadView& hv, int q_first, int kbase_, float c_) {
    lane = threadIdx.x & 63;
    const int col = lane & 31;
    half = lane >> 5;
    wq_first = q_first;
    wq_last = q_first + 31;
    my_q = q_first + col;
    kbase = kbase_;
    Sq = hv.Sq;
    Skv = hv.Skv;
    koff = hv.koff;
    c = c_;
    qsign = hv.qsign;
    // lane parts of the operand read addresses (the rest are immediates)
    k_lane = C::k_off(kbase + col) + half * 16;
    v_lane = C::v_off(kbase + 4 * half + ((lane & 15) >> 2)) + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
    if constexpr (LOAD_Q) {
      const __amdgpu_buffer_rsrc_t qr = make_rsrc(hv.q, rows_bytes(Sq, hv.q_ss, D));
      const uint32_t off = (uint32_t)(my_q * hv.q_ss + half * 8) * 2;  // rows >= Sq read 0
#pragma unroll
      for (int kc = 0; kc < DK; ++kc) qf[kc] = load16(qr, off + kc * 32) ^ qsign;
    }
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    m_run = -__builtin_inff();
    nm_ref = 0.f;
    m_thr = -__builtin_inff();
    l_run = 0.f;
    p_top = 0.f;
    e_top = 0.f;
    alpha = 1.f;
    pend_rs = false;
  }

  // Q through LDS.  Loaded straight into the fragment, a load instruction
  // reads 32 bytes from each of 32 rows; instead the wave copies its 32 rows
  // HBM -> LDS as whole rows (one copy instruction moves 1 KiB, Q_RPL
  // complete rows) and reads the fragment from there.  Line L of the area
  // (Q_LINES lines of 1 KiB + 16 bytes of padding) holds rows L, L + Q_LINES,
  // ..., so the 16-byte fragment reads of 8 consecutive rows hit distinct
  // banks.  Rows >= Sq read as 0.
  static constexpr int Q_RPL = 1024 / (2 * D);  // rows per line
  static constexpr int Q_LINES = 32 / Q_RPL;
  static constexpr int Q_LINE = 1024 + 16;
  static constexpr int Q_BYTES = Q_LINES * Q_LINE;
  __device__ __forceinline__ void copy_q(const HeadView& hv, uint8_t* area) const {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(hv.q, rows_bytes(Sq, hv.q_ss, D));
    const int m = lane / (D / 8), chunk = lane % (D / 8);
#pragma unroll
    for (int L = 0; L < Q_LINES; ++L)
      load16_lds(qr, area + L * Q_LINE, (uint32_t)((wq_first + L + Q_LINES * m) * hv.q_ss) * 2u + 16u * chunk);
  }
  __device__ __forceinline__ void read_q(const uint8_t* area) {
    const int col = lane & 31;
    const uint8_t* src = area + (col % Q_LINES) * Q_LINE + (col / Q_LINES) * (2 * D) + 16 * half;
#pragma unroll
    for (int kc = 0; kc < DK; ++kc) qf[kc] = *reinterpret_cast<const u32x4*>(src + 32 * kc) ^ qsign;
  }

  // P of a tile this wave skips: the next pv then adds exact zeros (and
  // owes O^T no rescale)
  __device__ __forceinline__ void zero_pf() {
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) pf[i] = u32x4{0u, 0u, 0u, 0u};
    alpha = 1.f;
    pend_rs = false;
  }

  // does this wave have any unmasked key in tile j?  Every operand is the
  // same in all lanes; readfirstlane lets the compiler see that too (in the
  // ping-pong kernel it had kept one in a VGPR and exec-masked the P = 0
  // moves of zero_pf(), issuing them on every tile)
  __device__ __forceinline__ bool active(int j) const {
    const int kv0 = j * BN + kbase;
    const bool a = kv0 < Skv && (!CAUSAL || kv0 <= wq_last + koff) && wq_first < Sq;
    return __builtin_amdgcn_readfirstlane((int)a) != 0;
  }

  __device__ __forceinline__ void qk(const uint8_t* kt) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < DK; ++kc) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kt + k_lane + C::k_off(32 * kb) + 32 * kc);
        sacc[kb] = E::mfma(a, qf[kc], sacc[kb]);
      }
    }
  }

  // DEFER_RESCALE leaves the rescale of O^T to the caller (rescale_o()
  // before the next pv), so that it can run next to MFMA work
  template <bool DEFER_RESCALE = false>
  __device__ __forceinline__ void softmax(int j) {
    const int kv0 = j * BN + kbase;
    // mask keys past the end or after the query (diagonal / ragged tiles).
    // The test is wave-uniform; in the ping-pong kernel readfirstlane makes
    // it a scalar branch (the compiler had exec-masked the mask there; A/B:
    // causal B=2 H=16 S=4096 bf16 126.5 -> 125.4 us), while kernel 1 at
    // D=256 ran 3 % slower that way and keeps the compiler's choice.
    const bool mask_test = (kv0 + C::KSUB > Skv) || (CAUSAL && kv0 + C::KSUB - 1 > wq_first + koff);
    const bool need_mask = C::PINGPONG ? __builtin_amdgcn_readfirstlane((int)mask_test) != 0 : mask_test;
    if (need_mask) {
      // score i of block kb is key kv0 + 4*half + off(kb, i); it is kept iff
      // key <= min(my_q + koff, Skv-1) (causal) or key <= Skv-1: one compare
      // of a constant offset against a per-lane limit
      const int last = CAUSAL ? (my_q + koff < Skv - 1 ? my_q + koff : Skv - 1) : Skv - 1;
      const int lim = last - kv0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
          sacc[kb][i] = off > lim ? -__builtin_inff() : sacc[kb][i];
        }
      }
    }

    // row max over this tile: a tree over the lane's 16*NB scores, then
    // across the lane pair
    float sc[16 * NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[16 * kb + i] = sacc[kb][i];
    const float mx = max_halves(max_tree<16 * NB>(sc));

    // Rescale only when some row's max outgrew the reference by the slack
    // (always on the first tile with an unmasked key, m_run being -inf
    // before); the branch is uniform across the wave.
    // c > 0, so a fully masked max stays -inf and never turns into NaN.
    const float mt = mx * c;
    if constexpr (DEFER_RESCALE) alpha = 1.f, pend_rs = false;
    if (__builtin_amdgcn_ballot_w64(mt > m_thr) != 0) {
      const float m_new = __builtin_elementwise_maximum(m_run, mt);
      const bool none = m_new == -__builtin_inff();
      const float a = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      nm_ref = none ? 0.f : -m_new;
      m_thr = m_new + kRescaleSlack;
      l_run *= a;
      p_top *= a;
      e_top *= a;
      if constexpr (DEFER_RESCALE) {
        alpha = a;
        pend_rs = true;
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= a;
      }
    }
    // P = exp2(c*s - m), rounded to nearest-even as the MFMA operand; the
    // fp32 row sum of the unrounded P feeds the LSE and, with e_top, O's
    // normaliser
    float ls[2 * NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float p[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * s2 + t], c, nm_ref));
        ls[2 * kb + s2] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pf[2 * kb + s2] = u32x4{E::pack2(p[0], p[1]), E::pack2(p[2], p[3]), E::pack2(p[4], p[5]),
                                E::pack2(p[6], p[7])};
      }
    }
#pragma unroll
    for (int w = 2 * NB; w > 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w / 2; ++i) ls[i] += ls[i + w / 2];
    l_run += ls[0];
    {
      // The largest P of this row in this tile, computed exactly as above,
      // and the error of its 16-bit rounding: the one of the row's largest P
      // so far joins O's normaliser (see e_top)
      const float pm = __builtin_amdgcn_exp2f(__builtin_fmaf(mx, c, nm_ref));
      const float em = E::round(pm) - pm;
      if (pm > p_top) p_top = pm, e_top = em;
    }
  }

  // O^T *= alpha: the rescale the last softmax asked for
  __device__ __forceinline__ void rescale_o() {
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
  }

  // O^T += V^T P^T.  MFMA k-slot t of this lane holds the key
  // 16*ks + 8*(t/4) + 4*half + t%4 (the score accumulator layout), so the
  // transposing read r = t/4 covers the 4 consecutive keys
  // 16*ks + 8*r + 4*half + (0..3) at d columns 32*db + (lane&31).
  __device__ __forceinline__ void pv(const uint8_t* vt) {
#pragma unroll
    for (int ks = 0; ks < 2 * NB; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint8_t* vp = vt + v_lane + 64 * db;
        const u32x2 lo = lds_read_tr16(vp + C::v_off(16 * ks));
        const u32x2 hi = lds_read_tr16(vp + C::v_off(16 * ks + 8));
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = E::mfma(a, pf[ks], oacc[db]);
      }
    }
  }

  // The MFMA work of one phase as one software pipeline: pv (O^T += V^T P^T
  // over the tile in vt) when PV, then qk (S^T = K Q^T over the tile in kt)
  // when QK.  Operand t+PIPE is read from LDS while MFMA t runs, and the
  // scheduling groups pin that interleave.  copy(i), i < NL, issues the i-th
  // HBM -> LDS copy instruction of the phase right after MFMA i*LSTRIDE, so
  // the copies queue up one at a time behind running MFMAs instead of
  // stalling the wave in a burst.
  template <bool PV, bool QK, int NL = 0, int LSTRIDE = 1, class COPY = NoCopy, int PIPE = 4>
  __device__ __forceinline__ void mfma_ops(const uint8_t* vt, const uint8_t* kt, const COPY& copy = COPY{}) {
    constexpr int NPV = PV ? 2 * NB * DB : 0;
    constexpr int NQK = QK ? DK * NB : 0;
    constexpr int NOPS = NPV + NQK;
    auto load = [&](int t) __attribute__((always_inline)) -> u32x4 {
      if (t < NPV) {
        const int ks = t / DB, db = t % DB;
        const uint8_t* vp = vt + v_lane + 64 * db;
        const u32x2 lo = lds_read_tr16(vp + C::v_off(16 * ks));
        const u32x2 hi = lds_read_tr16(vp + C::v_off(16 * ks + 8));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      const int t2 = t - NPV, kc = t2 / NB, kb = t2 % NB;
      return *reinterpret_cast<const u32x4*>(kt + k_lane + C::k_off(32 * kb) + 32 * kc);
    };
    u32x4 buf[PIPE];
#pragma unroll
    for (int t = 0; t < PIPE && t < NOPS; ++t) buf[t] = load(t);
#pragma unroll
    for (int t = 0; t < NOPS; ++t) {
      const u32x4 a = buf[t % PIPE];
      if (t + PIPE < NOPS) buf[t % PIPE] = load(t + PIPE);
      if (t < NPV) {
        const int ks = t / DB, db = t % DB;
        oacc[db] = E::mfma(a, pf[ks], oacc[db]);
      } else {
        const int t2 = t - NPV, kc = t2 / NB, kb = t2 % NB;
        sacc[kb] = E::mfma(a, qf[kc], kc == 0 ? f32x16{} : sacc[kb]);
      }
      if (NL > 0 && t % LSTRIDE == 0 && t / LSTRIDE < NL) copy(t / LSTRIDE);
    }
    static_assert(NL == 0 || (NL - 1) * LSTRIDE < NOPS, "copies must fit in the block");
    // desired order: the first PIPE operand reads, then MFMA t followed by
    // the reads of operand t+PIPE (and its copy)
    sched_prologue<0, NOPS, NPV, PIPE>();
    sched_steady<0, NOPS, NPV, PIPE, NL, LSTRIDE>();
  }

  // ---- kernel 3 (in-wave pipeline): explicit score and P arrays ----
  // MFMA slot block: qk (S^T = K Q^T over the tile in kt, into s) when QK,
  // then pv (O^T += V^T P^T over the tile in vt, with pp) when PV, as one
  // PIPE-deep operand pipeline.  After MFMA t come the reads of operand
  // t+PIPE, then this slot's share of the NL copy instructions (spread evenly
  // over the first LSLOTS slots) and of the NV VALU slices (over the first
  // VSLOTS slots); each slot is fenced from the next, so the instructions
  // stay in this order.  A wave issues in order: the VALU work placed between
  // its MFMAs runs while they execute.
  template <bool QK, bool PV, int NL, int LSLOTS, int NV, int VSLOTS, class COPY, class VALU, int PIPE = 4>
  __device__ __forceinline__ void mfma_slots(const uint8_t* kt, const uint8_t* vt, f32x16 (&s)[NB],
                                             const u32x4 (&pp)[2 * NB], const COPY& copy, const VALU& valu) {
    constexpr int NQK = QK ? DK * NB : 0;
    constexpr int NPV = PV ? 2 * NB * DB : 0;
    constexpr int NOPS = NQK + NPV;
    static_assert(LSLOTS >= 1 && LSLOTS <= NOPS && VSLOTS >= 1 && VSLOTS <= NOPS, "slots within the block");
    auto load = [&](int t) __attribute__((always_inline)) -> u32x4 {
      if (t < NQK) {
        const int kc = t / NB, kb = t % NB;
        return *reinterpret_cast<const u32x4*>(kt + k_lane + C::k_off(32 * kb) + 32 * kc);
      }
      const int t2 = t - NQK, ks = t2 / DB, db = t2 % DB;
      const uint8_t* vp = vt + v_lane + 64 * db;
      const u32x2 lo = lds_read_tr16(vp + C::v_off(16 * ks));
      const u32x2 hi = lds_read_tr16(vp + C::v_off(16 * ks + 8));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    // The wave's registers do not hold O, Q, two score and two P arrays at
    // once: the compiler parks some in AGPRs and, left alone, copies the Q
    // fragment back to VGPRs (four v_accvgpr_read per MFMA pair, ~60 VALU
    // instructions per iteration).  An MFMA reads its B operand from AGPRs
    // as well, so Q is pinned there and read in place (bit-identical; B=1
    // H=8 S=8192 D=256 causal 254.8 -> 246.7 us, B=1 H=16 S=4096 D=256
    // 247.8 -> 241.8 us).
    if constexpr (QK) {
#pragma unroll
      for (int kc = 0; kc < DK; ++kc) __asm__ volatile("" : "+a"(qf[kc]));
    }
    u32x4 buf[PIPE];
#pragma unroll
    for (int t = 0; t < PIPE && t < NOPS; ++t) buf[t] = load(t);
    // one instantiation per slot (the slices differ in kind, and a loop over
    // all of them is too large for the unroller)
    static_for<NOPS>([&](auto tc) __attribute__((always_inline)) {
      constexpr int t = decltype(tc)::value;
      const u32x4 a = buf[t % PIPE];
      if constexpr (t < NQK) {
        constexpr int kc = t / NB, kb = t % NB;
        s[kb] = E::mfma(a, qf[kc], kc == 0 ? f32x16{} : s[kb]);
      } else {
        constexpr int t2 = t - NQK, ks = t2 / DB, db = t2 % DB;
        oacc[db] = E::mfma(a, pp[ks], oacc[db]);
      }
      if constexpr (t + PIPE < NOPS) buf[t % PIPE] = load(t + PIPE);
      if constexpr (t < LSLOTS) {
        constexpr int l0 = t * NL / LSLOTS, l1 = (t + 1) * NL / LSLOTS;
        static_for<l1 - l0>([&](auto ic) __attribute__((always_inline)) { copy(l0 + decltype(ic)::value); });
      }
      if constexpr (t < VSLOTS) {
        constexpr int v0 = t * NV / VSLOTS, v1 = (t + 1) * NV / VSLOTS;
        static_for<v1 - v0>([&](auto ic) __attribute__((always_inline)) {
          valu(std::integral_constant<int, v0 + decltype(ic)::value>{});
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // softmax of one tile (scores s -> packed P pp, as softmax() computes them)
  // cut into NSLICES slices for mfma_slots: 0 masks, 1..NB take the row max
  // over score block kb and then across the lane pair, NB+1 decides the
  // rescale (O^T's own rescale is left to the caller: `pend` is set when
  // alpha != 1 for some lane), then one slice per pair of scores computes
  // and packs P with the pair's sum (a group of 8 scores completes its
  // partial sum in its fourth slice), and the last adds the tile's sum.
  struct SoftmaxState {
    float mx;
    float pe[8 * NB];  // pair sums
    float ls[2 * NB];  // 8-score group sums
  };
  static constexpr int NSLICES = 8 * NB + NB + 3;
  template <int sl>
  __device__ __forceinline__ void softmax_slice(int j, f32x16 (&s)[NB], u32x4 (&pp)[2 * NB], SoftmaxState& st,
                                                bool& pend) {
    if constexpr (sl == 0) {
      const int kv0 = j * BN + kbase;
      const bool need_mask = (kv0 + C::KSUB > Skv) || (CAUSAL && kv0 + C::KSUB - 1 > wq_first + koff);
      if (need_mask) {
        const int last = CAUSAL ? (my_q + koff < Skv - 1 ? my_q + koff : Skv - 1) : Skv - 1;
        const int lim = last - kv0 - 4 * half;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
            s[kb][i] = off > lim ? -__builtin_inff() : s[kb][i];
          }
      }
    } else if constexpr (sl <= NB) {
      constexpr int kb = sl - 1;
      float sc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = s[kb][i];
      const float m = max_tree<16>(sc);
      if constexpr (kb == 0)
        st.mx = m;
      else
        st.mx = __builtin_elementwise_maximum(st.mx, m);
      if constexpr (kb == NB - 1) st.mx = max_halves(st.mx);
      pin(st.mx);
    } else if constexpr (sl == NB + 1) {
      const float mt = st.mx * c;
      alpha = 1.f;
      pend = false;
      if (__builtin_amdgcn_ballot_w64(mt > m_thr) != 0) {
        const float m_new = __builtin_elementwise_maximum(m_run, mt);
        const bool none = m_new == -__builtin_inff();
        const float a = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        nm_ref = none ? 0.f : -m_new;
        m_thr = m_new + kRescaleSlack;
        l_run *= a;
        p_top *= a;
        e_top *= a;
        alpha = a;
        pend = true;
      }
    } else if constexpr (sl < NSLICES - 1) {
      constexpr int q = sl - (NB + 2);  // pair 0 .. 8NB-1
      constexpr int g = q / 4, pr = q % 4, kb = g / 2, s2 = g % 2;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * s2 + 2 * pr], c, nm_ref));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * s2 + 2 * pr + 1], c, nm_ref));
      pp[g][pr] = E::pack2(p0, p1);
      st.pe[q] = p0 + p1;
      pin(pp[g][pr]);
      pin(st.pe[q]);
      if constexpr (pr == 3) {
        st.ls[g] = (st.pe[q - 3] + st.pe[q - 2]) + (st.pe[q - 1] + st.pe[q]);
        pin(st.ls[g]);
      }
    } else {
#pragma unroll
      for (int w = 2 * NB; w > 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w / 2; ++i) st.ls[i] += st.ls[i + w / 2];
      l_run += st.ls[0];
      pin(l_run);
      const float pm = __builtin_amdgcn_exp2f(__builtin_fmaf(st.mx, c, nm_ref));
      const float em = E::round(pm) - pm;
      if (pm > p_top) p_top = pm, e_top = em;
      pin(p_top);
      pin(e_top);
    }
  }

  // O = O_acc / l (RNE to 16 bits), LSE = (m + log2 l) ln 2.
  // A row with no key (causal, Sq > Skv) has l = 0: O = 0 and LSE = -inf.
  // The accumulator layout gives each lane 8-byte pieces of its one row, so
  // a store instruction writes 16 bytes into each of 32 rows.
  __device__ __forceinline__ void epilogue(const HeadView& hv) {
    const float l_tot = sum_halves(l_run);
    if (my_q < Sq) {
      const float inv = l_tot > 0.f ? 1.0f / (l_tot + e_top) : 0.f;
      uint16_t* orow = hv.o + (int64_t)my_q * hv.o_ss;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * half;
          u32x2 w;
          w[0] = E::pack2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
          w[1] = E::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d) = w;
        }
      }
      if (half == 0)
        hv.lse[my_q] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
    }
  }

  // The same through LDS: the wave writes its 32 rows of O into `stage`
  // (EPI_BYTES of LDS that no other wave and no copy touches), reads them
  // back as whole rows and stores 16 contiguous bytes per lane, so one store
  // instruction covers 1024 / (2D) complete rows: 8x fewer memory requests
  // than the direct form.
  static constexpr int EPI_RS = 2 * D + 16;      // staged row stride (bytes)
  static constexpr int EPI_BYTES = 32 * EPI_RS;  // one wave's staging area
  __device__ __forceinline__ void epilogue_staged(const HeadView& hv, uint8_t* stage) {
    const float l_tot = sum_halves(l_run);
    const float inv = l_tot > 0.f ? 1.0f / (l_tot + e_top) : 0.f;
    uint8_t* mine = stage + (lane & 31) * EPI_RS;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * half;
        u32x2 w;
        w[0] = E::pack2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = E::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(mine + 2 * d) = w;
      }
    }
    // a wave's LDS accesses execute in order; keep the compiler from moving
    // the reads above the writes
    __asm__ volatile("" ::: "memory");
    constexpr int LPR = D / 8;     // lanes per row, 16 bytes each
    constexpr int RPI = 64 / LPR;  // rows per store instruction
    const int rl = lane / LPR, cl = lane % LPR;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + rl;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * EPI_RS + 16 * cl);
      if (wq_first + r < Sq)
        store_nt(v, reinterpret_cast<u32x4*>(hv.o + (int64_t)(wq_first + r) * hv.o_ss + 8 * cl));
    }
    if (my_q < Sq && half == 0)
      hv.lse[my_q] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
  }
};

// Staging areas of the staged epilogue: the K/V stage arrays, which no step
// reads once the key loop is over, cut into AREA-byte pieces in the order
// k0, k1, v0, v1 (array sizes NK0 .. NV1 bytes).  Piece w goes to wave w.
template <int AREA, int NK0, int NK1, int NV0, int NV1>
struct EpiAreas {
  static constexpr int P0 = NK0 / AREA, P1 = NK1 / AREA, P2 = NV0 / AREA, P3 = NV1 / AREA;
  static constexpr int TOTAL = P0 + P1 + P2 + P3;
  static __device__ __forceinline__ uint8_t* pick(int w, uint8_t* k0, uint8_t* k1, uint8_t* v0, uint8_t* v1) {
    if (w < P0) return k0 + w * AREA;
    w -= P0;
    if (w < P1) return k1 + w * AREA;
    w -= P1;
    if (w < P2) return v0 + w * AREA;
    return v1 + (w - P2) * AREA;
  }
};

// HBM -> LDS copies of K or V tiles of one head.  Line n of a tile holds rows
// (first row of line n) + STEP*m (STEP = KB for K, 4 for V); lane i of a copy
// instruction carries row STEP*(i / (D/8)) of the line and 16-byte chunk
// i % (D/8).  Rows at or past `rows` (the key length) fall outside the buffer
// descriptor and read as 0, as does a whole tile the caller marks invalid.
template <class C, bool IS_K>
struct TileCopier {
  static constexpr int D = C::D, STEP = IS_K ? C::KB : 4, LINE = IS_K ? C::K_LINE : C::V_LINE;
  const uint16_t* src;  // the head's first row
  int ss;               // row stride (elements)
  int rows;             // key length
  uint32_t lane_off;    // this lane's part of a line's source offset (bytes)

  __device__ __forceinline__ void init(const uint16_t* src_, int ss_, int rows_, int lane) {
    src = src_;
    ss = ss_;
    rows = rows_;
    lane_off = (uint32_t)(STEP * (lane / (D / 8)) * ss) * 2u + (uint32_t)(lane % (D / 8)) * 16u;
  }
  // descriptor over the rows of the tile that starts at key kv0
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile(int kv0, bool valid) const {
    return make_rsrc(src + (int64_t)kv0 * ss, (valid && kv0 < rows) ? rows_bytes(rows - kv0, ss, D) : 0u);
  }
  // the copy instruction of line ln of that tile into the LDS tile at dst
  __device__ __forceinline__ void line(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int ln) const {
    const int row0 = IS_K ? C::k_line_row(ln) : C::v_line_row(ln);
    load16_lds(r, dst + ln * LINE, lane_off, (uint32_t)(row0 * ss) * 2u);
  }
};

// Workgroup barrier that does not drain outstanding memory operations (the
// HBM -> LDS prefetch stays in flight).  The memory clobber keeps LDS accesses
// on their side; the scheduling fences keep register-only work (MFMAs, VALU)
// there too, which the clobber alone does not: without them the scheduler
// sinks the last MFMAs of a phase below the barrier, into the next phase.
__device__ __forceinline__ void barrier_keep_loads() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Wait for this wave's HBM -> LDS copies (vmcnt = 0).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's vector-memory operations are in flight
// (they complete in issue order): the older copies are then in LDS.
template <int N>
__device__ __forceinline__ void wait_loads_but() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N & 0x30) << 10));
}

// The end of kernels 1 and 3, after each wave's last read of the K/V stages:
// the key-split merge (KW > 1) and the output, staged through the stage
// arrays (stage arrays of one-stage shapes are 16-byte stand-ins).
template <class C, bool CAUSAL, int DT>
__device__ __forceinline__ void finish_tile(Wave<C, CAUSAL, DT>& w, const HeadView& hv, int qw, int kw, int lane,
                                            uint8_t* kt0, uint8_t* kt1, uint8_t* vt0, uint8_t* vt1) {
  constexpr int D = C::D, DB = C::DB;
  // Staged epilogue where the stage arrays hold a piece for every writing
  // wave (with a key split, only the kw = 0 waves write, and their pieces
  // must lie in the K arrays: with two or more stages the merge below reads
  // partials from V stages only; with one it uses kt0 too).
  using Areas = EpiAreas<Wave<C, CAUSAL, DT>::EPI_BYTES, C::K_TILE, C::STAGES >= 2 ? C::K_TILE : 16, C::V_TILE,
                         C::STAGES >= 2 ? C::V_TILE : 16>;
  constexpr bool STAGED = C::KW == 1 ? Areas::TOTAL >= C::NW
                                     : (C::STAGES >= 2 && (C::KW - 1) * C::QW <= 2 && Areas::P0 + Areas::P1 >= C::QW);
  wait_loads();  // the (empty) copies issued past the last tile
  // the key-split merge and the staged epilogue reuse the stage arrays: every
  // wave's copies must have landed before any wave writes there
  if constexpr (C::KW > 1 || STAGED) __syncthreads();

  // merge the key-split waves (KW > 1): the O partial of wave (kw, qw),
  // kw > 0, goes to slot (kw - 1) * QW + qw of the stage arrays (vt0, vt1,
  // kt0, kt1 with two or more stages; vt0, kt0 with one), its l, m, p_top
  // and e_top to a small array of their own
  if constexpr (C::KW > 1) {
    constexpr int NSLOT = (C::KW - 1) * C::QW;
    constexpr int SLOTS = C::STAGES >= 2 ? 4 : 2;
    constexpr int OBYTES = D / 2 * 64 * 4;  // one wave's O partial
    static_assert(NSLOT <= SLOTS && OBYTES <= C::V_TILE && (NSLOT <= SLOTS / 2 || OBYTES <= C::K_TILE),
                  "merge area too small");
    __shared__ float mscal[NSLOT][4][64];
    auto slot = [&](int i) __attribute__((always_inline)) -> uint8_t* {
      if constexpr (SLOTS == 2) return i == 0 ? vt0 : kt0;
      return i == 0 ? vt0 : i == 1 ? vt1 : i == 2 ? kt0 : kt1;
    };
    if (kw > 0) {
      const int sl = (kw - 1) * C::QW + qw;
      float* dst = reinterpret_cast<float*>(slot(sl));
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(db * 16 + i) * 64 + lane] = w.oacc[db][i];
      mscal[sl][0][lane] = w.l_run;
      mscal[sl][1][lane] = w.m_run;
      mscal[sl][2][lane] = w.p_top;
      mscal[sl][3][lane] = w.e_top;
    }
    __syncthreads();
    if (kw > 0) return;
#pragma unroll
    for (int ww = 1; ww < C::KW; ++ww) {
      const int sl = (ww - 1) * C::QW + qw;
      const float* src = reinterpret_cast<const float*>(slot(sl));
      const float lb = mscal[sl][0][lane];
      const float mb = mscal[sl][1][lane];
      const float pb = mscal[sl][2][lane];
      const float eb = mscal[sl][3][lane];
      const float mm = fmaxf(w.m_run, mb);
      const float mref = (mm == -__builtin_inff()) ? 0.f : mm;
      const float fa = __builtin_amdgcn_exp2f(w.m_run - mref);
      const float fb = __builtin_amdgcn_exp2f(mb - mref);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          w.oacc[db][i] = w.oacc[db][i] * fa + src[(db * 16 + i) * 64 + lane] * fb;
      w.l_run = w.l_run * fa + lb * fb;
      // the larger of the two largest P, on the merged scale, with its error
      const float pa = w.p_top * fa, pbs = pb * fb;
      w.e_top = pa >= pbs ? w.e_top * fa : eb * fb;
      w.p_top = pa >= pbs ? pa : pbs;
      w.m_run = mm;
    }
  }

  if constexpr (STAGED)
    w.epilogue_staged(hv, Areas::pick(qw, kt0, kt1, vt0, vt1));
  else
    w.epilogue(hv);
}

// ---------------------------------------------------------------------------
// Kernel 1: every wave runs qk, softmax, pv per tile.  Copy schedules:
//   STAGGER (two LDS stages of K and of V): every copy gets about a tile and
//   a half to land, for workgroups that are alone on their CU (D=256):
//     qk(j)      carries the copy of V_{j+1} (into the V stage pv(j-1) freed)
//     softmax(j)
//     wait V_j, barrier
//     pv(j)      carries the copy of K_{j+2} (into the K stage qk(j) freed)
//     wait K_{j+1}, barrier
//   (the copy instructions ride in the MFMA blocks, one after every few MFMAs);
//   otherwise STAGES = 2: K_{j+1} and V_{j+1} are copied while tile j is
//   computed, with one barrier per tile, where several workgroups share a CU
//   and cover each other's copy latency (D=64: four per CU); STAGES = 1 or 3
//   (and a producer wave) serve the schedule variants.
// Supports key-split waves (KW > 1), merged at the end through LDS.
// ---------------------------------------------------------------------------
template <class C, bool CAUSAL, int DT>
__global__ __launch_bounds__(C::NT) void attn_fwd_kernel(const Problem p) {
  constexpr int BN = C::BN, BM = C::BM, DB = C::DB;
  constexpr int LPW = C::LINES / C::NW;              // copy lines per wave per operand
  constexpr int NQK = C::DK * C::NB, NPV = 2 * C::NB * DB;  // MFMAs of qk, pv
  constexpr int LSQ = NQK / LPW, LSP = NPV / LPW;      // MFMAs per copy
  static_assert(LSQ >= 1 && LSP >= 1, "copies must fit in the MFMA blocks");

  // one array per stage and operand, so that the compiler can tell reads of
  // one stage from the asynchronous HBM->LDS copies into the other
  __shared__ __attribute__((aligned(1024))) uint8_t kt0[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kt1[C::STAGES >= 2 ? C::K_TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t kt2[C::STAGES >= 3 ? C::K_TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vt0[C::V_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vt1[C::STAGES >= 2 ? C::V_TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vt2[C::STAGES >= 3 ? C::V_TILE : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qw = wave % C::QW;
  const int kw = wave / C::QW;
  // the copying wave of a PRODUCER workgroup (wave NW) computes nothing
  const bool producer = C::PRODUCER && wave == C::NW;

  uint32_t tile, bh;
  workgroup_tile<CAUSAL>(p.map, blockIdx.x, &tile, &bh);
  const int q0 = (int)tile * BM;
  const HeadView hv = head_view(p, bh);

  // Q through LDS where a second K/V stage exists: the loop's first iteration
  // writes it (the staggered schedule: vt1 only), so the waves stage their Q
  // rows there first, one slice per query wave shared by its key waves
  using W = Wave<C, CAUSAL, DT>;
  constexpr int QPK = C::K_TILE / W::Q_BYTES, QPV = C::V_TILE / W::Q_BYTES;  // slices per array
  constexpr bool STAGE_Q = !C::PRODUCER && C::STAGES == 2 && (C::STAGGER ? QPV >= C::QW : QPK + QPV >= C::QW);
  W w;
  if (!producer) w.template init<!STAGE_Q>(hv, q0 + qw * 32, kw * C::KSUB, p.c);
  uint8_t* const q_area =
      C::STAGGER ? vt1 + qw * W::Q_BYTES : (qw < QPK ? kt1 + qw * W::Q_BYTES : vt1 + (qw - QPK) * W::Q_BYTES);
  // after the copies of the first tiles (and the barrier that ends them):
  // every wave reads its fragment, and a second barrier keeps the loop's
  // copies into those arrays behind all the reads
  auto read_staged_q = [&]() __attribute__((always_inline)) {
    if constexpr (STAGE_Q) {
      w.read_q(q_area);
      __syncthreads();
    }
  };

  // key tiles this workgroup needs (none when causal leaves its rows no key)
  const int q_end = (q0 + BM < hv.Sq) ? q0 + BM : hv.Sq;
  const int kv_end = CAUSAL ? (q_end + hv.koff < 0 ? 0 : (q_end + hv.koff < hv.Skv ? q_end + hv.koff : hv.Skv))
                            : hv.Skv;
  const int n = (kv_end + BN - 1) / BN;
  if (n == 0) {  // uniform over the workgroup
    if (!producer) w.epilogue(hv);
    return;
  }

  // a tile past the last one this workgroup needs reads through an empty
  // descriptor (no fetch; it fills a stage no later step reads)
  TileCopier<C, true> kcp;
  TileCopier<C, false> vcp;
  kcp.init(hv.k, hv.k_ss, hv.Skv, lane);
  vcp.init(hv.v, hv.v_ss, hv.Skv, lane);
  auto k_copier = [&](int t, uint8_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = kcp.tile(t * BN, t < n);
    return [=](int i) __attribute__((always_inline)) { kcp.line(r, dst, wave * LPW + i); };
  };
  auto v_copier = [&](int t, uint8_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = vcp.tile(t * BN, t < n);
    return [=](int i) __attribute__((always_inline)) { vcp.line(r, dst, wave * LPW + i); };
  };

  if constexpr (C::STAGGER) {
    // tile j: K_j in kt_j, V_j in vt_j; vt_o is the other V stage
    auto iter = [&](int j, uint8_t* kt_j, uint8_t* vt_j, uint8_t* vt_o) __attribute__((always_inline)) {
      const bool act = w.active(j);
      const auto cv = v_copier(j + 1, vt_o);
      if (act) {
        w.template mfma_ops<false, true, LPW, LSQ>(vt_j, kt_j, cv);
        w.softmax(j);
      } else {
#pragma unroll
        for (int i = 0; i < LPW; ++i) cv(i);
      }
      wait_loads_but<2 * LPW>();  // V_j landed (K_{j+1}, V_{j+1} may still be in flight)
      barrier_keep_loads();       // V_j complete in LDS; every wave is done with kt_j
      const auto ck = k_copier(j + 2, kt_j);
      if (act) {
        w.template mfma_ops<true, false, LPW, LSP>(vt_j, kt_j, ck);
      } else {
#pragma unroll
        for (int i = 0; i < LPW; ++i) ck(i);
      }
      wait_loads_but<2 * LPW>();  // K_{j+1} landed (V_{j+1}, K_{j+2} may still be in flight)
      barrier_keep_loads();       // K_{j+1} complete in LDS; every wave is done with vt_j
    };
    {
      const auto k0 = k_copier(0, kt0);
      const auto v0 = v_copier(0, vt0);
      const auto k1 = k_copier(1, kt1);
#pragma unroll
      for (int i = 0; i < LPW; ++i) k0(i), v0(i), k1(i);
    }
    if (STAGE_Q && kw == 0) w.copy_q(hv, q_area);
    wait_loads();
    __syncthreads();
    read_staged_q();
    for (int j = 0; j < n; j += 2) {
      iter(j, kt0, vt0, vt1);
      if (j + 1 < n) iter(j + 1, kt1, vt1, vt0);
    }
  } else {
    // copies of tile t (empty past the last tile) into (kt, vt): LPW lines of
    // K and of V per wave, or all of them by the producer wave
    constexpr int CPT = C::PRODUCER ? 2 * C::LINES : 2 * LPW;  // copy instructions per tile, copying wave
    auto fetch = [&](int t, uint8_t* kt, uint8_t* vt) __attribute__((always_inline)) {
      if constexpr (C::PRODUCER) {
        if (!producer) return;
        const auto ck = k_copier(t, kt);
        const auto cv = v_copier(t, vt);
        // the copiers address line wave * LPW + i, and the producer is wave NW
#pragma unroll
        for (int i = 0; i < C::LINES; ++i) ck(i - C::NW * LPW), cv(i - C::NW * LPW);
      } else {
        const auto ck = k_copier(t, kt);
        const auto cv = v_copier(t, vt);
#pragma unroll
        for (int i = 0; i < LPW; ++i) ck(i), cv(i);
      }
    };
    auto compute = [&](int j, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
      if (producer || !w.active(j)) return;
      w.qk(kt);
      w.softmax(j);
      w.pv(vt);
    };
    if constexpr (C::STAGES == 1) {
      // copy, wait, compute, and wait until every wave is done reading
      for (int j = 0; j < n; ++j) {
        fetch(j, kt0, vt0);
        __syncthreads();
        compute(j, kt0, vt0);
        __syncthreads();
      }
    } else if constexpr (C::STAGES == 2) {
      // tile j+1 is copied while tile j is computed; one barrier per tile
      fetch(0, kt0, vt0);
      if (STAGE_Q && kw == 0) w.copy_q(hv, q_area);
      __syncthreads();
      read_staged_q();
      for (int j = 0; j < n; j += 2) {
        if (j + 1 < n) fetch(j + 1, kt1, vt1);
        compute(j, kt0, vt0);
        __syncthreads();
        if (j + 1 < n) {
          if (j + 2 < n) fetch(j + 2, kt0, vt0);
          compute(j + 1, kt1, vt1);
          __syncthreads();
        }
      }
    } else {
      // tile j+2 is copied while tile j is computed, so every copy has two
      // tiles' time to land; the counted wait lets tile j+2's copies stay in
      // flight (tiles past the end are empty copies, so the count is uniform)
      fetch(0, kt0, vt0);
      fetch(1, kt1, vt1);
      wait_loads_but<CPT>();
      barrier_keep_loads();
      auto step = [&](int j, const uint8_t* kt, const uint8_t* vt, uint8_t* kn, uint8_t* vn)
                      __attribute__((always_inline)) {
        fetch(j + 2, kn, vn);
        compute(j, kt, vt);
        wait_loads_but<CPT>();  // tile j+1 landed
        barrier_keep_loads();
      };
      for (int j = 0; j < n; j += 3) {
        step(j, kt0, vt0, kt2, vt2);
        if (j + 1 < n) step(j + 1, kt1, vt1, kt0, vt0);
        if (j + 2 < n) step(j + 2, kt2, vt2, kt1, vt1);
      }
    }
  }
  if (producer) {
    wait_loads();
    return;
  }
  finish_tile(w, hv, qw, kw, lane, kt0, kt1, vt0, vt1);
}

// ---------------------------------------------------------------------------
// Kernel 2 (ping-pong): 8 waves in two groups of 4, one wave of each group
// per SIMD (waves w and w+4 share a SIMD).  The SIMD overlaps one wave's MFMAs
// with another wave's VALU instructions, so time is cut into phases X_j, Y_j
// separated by workgroup barriers, and in each phase one group issues MFMA
// work while the other issues VALU work:
//   X_j: group 0 pv(j-1), qk(j)      group 1 softmax(j-1)
//   Y_j: group 0 softmax(j)          group 1 pv(j-1), qk(j)
// Both groups run the loop body [pv(j-1), qk(j)] barrier [softmax(j)]
// barrier, j = 0..n (n key tiles); group 1 starts one phase later.  The
// first iteration has no pv and the last (j = n) no qk and no softmax; in
// between the MFMA half is one straight-line block, and a tile a wave does
// not need gets P = 0, so its pv adds exact zeros.  K and V tiles rotate
// through three LDS stages when they fit, else two.  Group 0 copies them:
// its MFMA block in X_j carries the copy instructions of K_{j+ST-1} and
// V_{j+ST-2}, one after every few MFMAs, and before the barrier that ends
// Y_j it waits for the copies that X_{j+1} reads (three stages: those of the
// previous iteration; two: those of this one).  Copies past the last tile
// read through an empty buffer descriptor: they fetch nothing and fill a
// stage no later phase reads.  With two stages each group writes its output
// inside the last iteration, right after its last pv (group 0 during Y_n).
// ---------------------------------------------------------------------------
// MFMAs between two copy instructions in group 0's MFMA block
constexpr int kPingPongCopyStride = 3;
// Whether the ping-pong rescales O^T (when a row max moved past the slack) at
// the start of the next MFMA phase instead of in the softmax phase.  Deferred
// is faster: the softmax phase is the longer one, and with the multiplies
// there the compiler spilled registers of the causal kernel.  The multiplies
// run only on a wave-uniform flag: with the lagging max few wave-tiles need
// them, and issued on every tile (alpha = 1) they were 64 VALU instructions
// per tile beside the MFMAs in a kernel whose clock the power limit sets.
constexpr bool kPingPongDeferRescale = true;
template <class C, bool CAUSAL, int DT>
__global__ __launch_bounds__(C::NT) void attn_fwd_pingpong_kernel(const Problem p) {
  static_assert(C::NW == 8 && C::KW == 1, "ping-pong needs 8 query waves");
  constexpr int BN = C::BN, BM = C::BM;
  constexpr int LPW = C::LINES / 4;  // copy instructions per loading wave and operand
  constexpr int ST = 3 * (C::K_TILE + C::V_TILE) <= 160 * 1024 ? 3 : 2;  // LDS stages
  static_assert(2 * (C::K_TILE + C::V_TILE) <= 160 * 1024, "two stages must fit in LDS");
  constexpr int T3 = ST == 3 ? 1 : 0;

  __shared__ __attribute__((aligned(1024))) uint8_t kt0[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kt1[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kt2[T3 ? C::K_TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vt0[C::V_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vt1[C::V_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vt2[T3 ? C::V_TILE : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = wave >> 2;

  uint32_t tile, bh;
  workgroup_tile<CAUSAL>(p.map, blockIdx.x, &tile, &bh);
  const int q0 = (int)tile * BM;
  const HeadView hv = head_view(p, bh);

  // with two stages the V stage arrays are free until the first iteration
  // copies V_0: the waves stage their Q rows there
  constexpr bool STAGE_Q = ST == 2 && 4 * Wave<C, CAUSAL, DT>::Q_BYTES <= C::V_TILE;
  Wave<C, CAUSAL, DT> w;
  w.template init<!STAGE_Q>(hv, q0 + wave * 32, 0, p.c);

  // key tiles this workgroup needs (none when causal leaves its rows no key)
  const int q_end = (q0 + BM < hv.Sq) ? q0 + BM : hv.Sq;
  const int kv_end = CAUSAL ? (q_end + hv.koff < 0 ? 0 : (q_end + hv.koff < hv.Skv ? q_end + hv.koff : hv.Skv))
                            : hv.Skv;
  const int n = (kv_end + BN - 1) / BN;
  if (n == 0) {  // uniform over the workgroup
    w.epilogue(hv);
    return;
  }

  TileCopier<C, true> kcp;
  TileCopier<C, false> vcp;
  kcp.init(hv.k, hv.k_ss, hv.Skv, lane);
  vcp.init(hv.v, hv.v_ss, hv.Skv, lane);

  // With two stages the output leaves inside the last iteration (j = n,
  // pv(n-1) only): group 0 stages its rows in the K arrays during Y_n, while
  // group 1 runs its last pv, and group 1 stages its rows in the V array
  // that holds no tile any more, right after that pv.  No K array is read or
  // copied into after Y_{n-1}, and the free V array last held V_{n-2}.
  constexpr bool EARLY_OUT = ST == 2;
  using W = Wave<C, CAUSAL, DT>;
  using KAreas = EpiAreas<W::EPI_BYTES, C::K_TILE, C::K_TILE, 0, 0>;
  static_assert(!EARLY_OUT || (KAreas::TOTAL >= 4 && 4 * W::EPI_BYTES <= C::V_TILE),
                "a group's output must fit the K arrays and one V array");

  // One iteration of this wave.  PV, QK select the halves of the MFMA block;
  // group 0 (COPIES) also copies the next tiles.  kt_j holds K_j, vt_prev
  // holds V_{j-1}; the copies of K_{j+ST-1} and V_{j+ST-2} go to kt_ld and
  // vt_ld.  The stages of iterations that copy are always named arrays: the
  // compiler keeps apart LDS reads and in-flight copies only by their array.
  auto iter = [&](auto copies, auto pv, auto qk, int j, const uint8_t* kt_j, uint8_t* kt_ld, uint8_t* vt_ld,
                  const uint8_t* vt_prev) __attribute__((always_inline)) {
    constexpr bool COPIES = decltype(copies)::value;
    constexpr bool PV = decltype(pv)::value, QK = decltype(qk)::value;
    constexpr bool LAST = !QK;  // j = n: pv(n-1) only
    if constexpr (COPIES && !LAST) {
      const __amdgpu_buffer_rsrc_t rk = kcp.tile((j + ST - 1) * BN, j + ST - 1 < n);
      const __amdgpu_buffer_rsrc_t rv = vcp.tile((j + ST - 2) * BN, j + ST - 2 < n);
      auto copy = [&](int i) __attribute__((always_inline)) {
        if (i < LPW)
          kcp.line(rk, kt_ld, wave * LPW + i);
        else
          vcp.line(rv, vt_ld, wave * LPW + i - LPW);
      };
      constexpr int LS = (PV && QK) ? kPingPongCopyStride : 2;
      if constexpr (kPingPongDeferRescale && PV) {
        if (w.pend_rs) w.rescale_o();
      }
      w.template mfma_ops<PV, QK, 2 * LPW, LS>(vt_prev, kt_j, copy);
    } else {
      if constexpr (kPingPongDeferRescale && PV) {
        if (w.pend_rs) w.rescale_o();
      }
      w.template mfma_ops<PV, QK>(vt_prev, kt_j);
    }
    barrier_keep_loads();
    if constexpr (!LAST) {
      if (w.active(j)) w.template softmax<kPingPongDeferRescale>(j);
      else w.zero_pf();
    }
    if constexpr (COPIES) {
      if constexpr (ST == 3 && !LAST) wait_loads_but<2 * LPW>();  // the previous iteration's copies landed
      else wait_loads();
    }
    if (COPIES || !LAST) barrier_keep_loads();
  };
  // the last iteration with two stages: pv(n-1) from vt_prev, then the
  // output (vt_free is the V array without a tile)
  auto last = [&](auto copies, const uint8_t* vt_prev, uint8_t* vt_free) __attribute__((always_inline)) {
    if constexpr (kPingPongDeferRescale) {
      if (w.pend_rs) w.rescale_o();
    }
    w.template mfma_ops<true, false>(vt_prev, kt0);
    if constexpr (decltype(copies)::value) {
      barrier_keep_loads();  // end of X_n
      w.epilogue_staged(hv, KAreas::pick(wave, kt0, kt1, kt0, kt0));
    } else {
      w.epilogue_staged(hv, vt_free + (wave & 3) * W::EPI_BYTES);
    }
    barrier_keep_loads();  // end of Y_n
  };
  auto loop = [&](auto copies) __attribute__((always_inline)) {
    using Y = std::true_type;
    using N = std::false_type;
    // stages of iteration j: kt[j % ST], kt[(j+ST-1) % ST], vt[(j+ST-2) % ST], vt[(j+ST-1) % ST]
    if constexpr (ST == 3) {
      iter(copies, N{}, Y{}, 0, kt0, kt2, vt1, vt2);
      for (int j = 1; j < n; j += 3) {
        iter(copies, Y{}, Y{}, j, kt1, kt0, vt2, vt0);
        if (j + 1 < n) iter(copies, Y{}, Y{}, j + 1, kt2, kt1, vt0, vt1);
        if (j + 2 < n) iter(copies, Y{}, Y{}, j + 2, kt0, kt2, vt1, vt2);
      }
      const int r = (n - 1) % 3;
      iter(copies, Y{}, N{}, n, kt0, kt0, vt0, r == 0 ? vt0 : (r == 1 ? vt1 : vt2));
    } else {
      iter(copies, N{}, Y{}, 0, kt0, kt1, vt0, vt1);
      for (int j = 1; j < n; j += 2) {
        iter(copies, Y{}, Y{}, j, kt1, kt0, vt1, vt0);
        if (j + 1 < n) iter(copies, Y{}, Y{}, j + 1, kt0, kt1, vt0, vt1);
      }
      last(copies, (n & 1) ? vt0 : vt1, (n & 1) ? vt1 : vt0);
    }
  };

  uint8_t* const q_area = (wave < 4 ? vt0 : vt1) + (wave & 3) * Wave<C, CAUSAL, DT>::Q_BYTES;
  if constexpr (STAGE_Q) w.copy_q(hv, q_area);
  if (group == 0) {
    const __amdgpu_buffer_rsrc_t rk0 = kcp.tile(0, true);
#pragma unroll
    for (int i = 0; i < LPW; ++i) kcp.line(rk0, kt0, wave * LPW + i);
    if constexpr (ST == 3) {
      const __amdgpu_buffer_rsrc_t rk1 = kcp.tile(BN, n > 1);
      const __amdgpu_buffer_rsrc_t rv0 = vcp.tile(0, true);
#pragma unroll
      for (int i = 0; i < LPW; ++i) kcp.line(rk1, kt1, wave * LPW + i), vcp.line(rv0, vt0, wave * LPW + i);
    }
  }
  wait_loads();
  __syncthreads();
  if constexpr (STAGE_Q) {
    w.read_q(q_area);
    __syncthreads();  // every wave holds its Q before V_0 is copied over the areas
  }
  if (group == 0) {
    loop(std::true_type{});
  } else {
    barrier_keep_loads();  // group 1 idles through X_0
    loop(std::false_type{});
  }

  if constexpr (!EARLY_OUT) {
    // the loop's last barrier has passed: every wave is done with LDS
    using Areas = EpiAreas<W::EPI_BYTES, C::K_TILE, C::K_TILE, C::V_TILE, C::V_TILE>;
    static_assert(Areas::TOTAL >= 8, "the staged epilogue needs a piece per wave");
    w.epilogue_staged(hv, Areas::pick(wave, kt0, kt1, vt0, vt1));
  }
}

// ---------------------------------------------------------------------------
// Kernel 3 (in-wave pipeline): one wave per SIMD, each wave alone with the
// matrix core of its SIMD, so the overlap of MFMA and VALU work comes from
// the wave's own instruction stream.  Iteration j of a wave issues
//   MFMAs: qk(j+1) into the other score array, then pv(j-1)
//   VALU:  softmax(j) (score array of tile j -> packed P of tile j), in
//          slices placed between those MFMAs
// and waits for its copies of K_{j+2} and V_j, then meets the other waves at
// one barrier.  The rescale of O^T that softmax(j) may ask for runs at the
// start of iteration j+1, before pv(j).  Tile t's K and V live in stage
// t % 2; the copies of iteration j go to the stages that iteration j-1 was
// the last to read.  Score and P arrays alternate between two named sets, so
// the loop is unrolled by two.
// ---------------------------------------------------------------------------
// D = 256 shape choice: the in-wave kernel's 128-row query tiles where the
// grid holds at least two rounds of them for a 256-CU part; smaller grids
// take 64-row tiles (kernel 1, twice the workgroups).  Measured on MI355X:
// the 128-row tiles are 12-15 % faster at 1x8x8192 causal and 1x16x4096,
// but slower where they leave CUs idle or long causal tiles set the end
// (1x16x2048 causal 61 against 51 us, 2x8x1024 31 against 25 us).
constexpr int64_t kInwaveMinWorkgroups = 512;
__host__ __device__ inline bool use_inwave_256(int64_t BH, int64_t S) {
  return BH * ((S + 127) / 128) >= kInwaveMinWorkgroups;
}

// The copies of an iteration go out over its first half of MFMA slots (each
// copy then has over half an iteration to land; over all the slots the
// iteration took 5 % longer, over the first eighth 4 %, over the first
// quarter or third 0.2-1.3 %), the softmax slices over all of them (packed
// into the first two thirds: 1-3 % slower).
constexpr int kInwaveCopyDiv = 2;
template <class C, bool CAUSAL, int DT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::D <= 128 ? 2 : 1)))
void attn_fwd_inwave_kernel(const Problem p) {
  static_assert(C::INWAVE && C::NW == 4, "the in-wave pipeline runs 4 waves, one per SIMD");
  constexpr int BN = C::BN, BM = C::BM, NB = C::NB;
  constexpr int LPW = C::LINES / C::NW;  // copy lines per wave per operand
  using W = Wave<C, CAUSAL, DT>;

  __shared__ __attribute__((aligned(1024))) uint8_t kt0[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kt1[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vt0[C::V_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vt1[C::V_TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qw = wave % C::QW, kw = wave / C::QW;

  uint32_t tile, bh;
  workgroup_tile<CAUSAL>(p.map, blockIdx.x, &tile, &bh);
  const int q0 = (int)tile * BM;
  const HeadView hv = head_view(p, bh);

  // Q through the V stages, which the loop's first copies only reach after
  // the barrier that follows qk(0): the kw = 0 waves copy the rows of their
  // query wave, every wave reads its fragment
  constexpr int QPV = C::V_TILE / W::Q_BYTES;  // query waves' rows per V stage
  static_assert(2 * QPV >= C::QW, "the Q rows must fit in the V stages");
  W w;
  w.template init<false>(hv, q0 + qw * 32, kw * C::KSUB, p.c);

  const int q_end = (q0 + BM < hv.Sq) ? q0 + BM : hv.Sq;
  const int kv_end = CAUSAL ? (q_end + hv.koff < 0 ? 0 : (q_end + hv.koff < hv.Skv ? q_end + hv.koff : hv.Skv))
                            : hv.Skv;
  const int n = (kv_end + BN - 1) / BN;
  uint8_t* const q_area = (qw < QPV ? vt0 + qw * W::Q_BYTES : vt1 + (qw - QPV) * W::Q_BYTES);
  if (n == 0) {  // uniform over the workgroup: no key for any row
    if (kw == 0) w.epilogue(hv);
    return;
  }

  TileCopier<C, true> kcp;
  TileCopier<C, false> vcp;
  kcp.init(hv.k, hv.k_ss, hv.Skv, lane);
  vcp.init(hv.v, hv.v_ss, hv.Skv, lane);
  {
    const __amdgpu_buffer_rsrc_t r0 = kcp.tile(0, true), r1 = kcp.tile(BN, n > 1);
#pragma unroll
    for (int i = 0; i < LPW; ++i) kcp.line(r0, kt0, wave * LPW + i), kcp.line(r1, kt1, wave * LPW + i);
  }
  if (kw == 0) w.copy_q(hv, q_area);
  wait_loads();
  __syncthreads();
  w.read_q(q_area);

  f32x16 s0[NB], s1[NB];
  u32x4 p0[2 * NB], p1[2 * NB];
  bool pend = false;
  auto no_copy = [](int) {};
  auto no_valu = [](auto) {};
  // qk(0), alone; the barrier after it frees kt0 and the Q areas for copies
  w.template mfma_slots<true, false, 0, 1, 0, 1>(kt0, vt0, s0, p1, no_copy, no_valu);
  barrier_keep_loads();

  auto iter = [&](auto pv, int j, f32x16(&s_cur)[NB], u32x4(&p_cur)[2 * NB], f32x16(&s_next)[NB],
                  const u32x4(&p_prev)[2 * NB], const uint8_t* kt_qk, const uint8_t* vt_pv, uint8_t* kt_ld,
                  uint8_t* vt_ld) __attribute__((always_inline)) {
    constexpr bool PV = decltype(pv)::value;
    if constexpr (PV) {
      if (pend) w.rescale_o();  // softmax(j-1)'s rescale, before pv(j-1)
    }
    const __amdgpu_buffer_rsrc_t rk = kcp.tile((j + 2) * BN, j + 2 < n);
    const __amdgpu_buffer_rsrc_t rv = vcp.tile(j * BN, true);
    auto copy = [&](int i) __attribute__((always_inline)) {
      if (i < LPW)
        kcp.line(rk, kt_ld, wave * LPW + i);
      else
        vcp.line(rv, vt_ld, wave * LPW + i - LPW);
    };
    typename W::SoftmaxState st;
    auto valu = [&](auto sl) __attribute__((always_inline)) {
      w.template softmax_slice<decltype(sl)::value>(j, s_cur, p_cur, st, pend);
    };
    constexpr int NS = C::DK * NB + (PV ? 2 * NB * C::DB : 0);  // MFMA slots (the first iteration: qk only)
    constexpr int LS = NS / kInwaveCopyDiv, VS = NS;
    w.template mfma_slots<true, PV, 2 * LPW, LS, W::NSLICES, VS>(kt_qk, vt_pv, s_next, p_prev, copy, valu);
    wait_loads();  // K_{j+2} and V_j landed
    barrier_keep_loads();
  };

  using Y = std::true_type;
  using N = std::false_type;
  iter(N{}, 0, s0, p0, s1, p1, kt1, vt1, kt0, vt0);
  for (int j = 1; j < n; j += 2) {
    iter(Y{}, j, s1, p1, s0, p0, kt0, vt0, kt1, vt1);
    if (j + 1 < n) iter(Y{}, j + 1, s0, p0, s1, p1, kt1, vt1, kt0, vt0);
  }
  // pv(n-1)
  if (pend) w.rescale_o();
  if ((n - 1) & 1)
    w.template mfma_slots<false, true, 0, 1, 0, 1>(kt1, vt1, s0, p1, no_copy, no_valu);
  else
    w.template mfma_slots<false, true, 0, 1, 0, 1>(kt0, vt0, s0, p0, no_copy, no_valu);
  finish_tile(w, hv, qw, kw, lane, kt0, kt1, vt0, vt1);
}

}  // namespace attn
