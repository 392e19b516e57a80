// attn_bwd.hpp -- host-side view of the backward kernels: the problem they
// read and the launcher that plans and enqueues them (attn_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_grid.hpp"

namespace attn {

// Batch, head and row strides (elements) of one [B,H,rows,D] tensor whose
// rows are contiguous.
struct Strides {
  int64_t sb, sh;
  int ss;
};

// Q, O, dO, dQ [B,H,Sq,D] and K, V, dK, dV [B,H,Skv,D] of 16-bit elements,
// each with its own strides; LSE and delta [B,H,Sq] fp32, contiguous.  Causal
// keeps key j for query i iff j <= i + (Skv - Sq), as in the forward.
struct BwdProblem {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dO;
  const float* lse;
  float* delta;  // written by the dQ kernel (run first): D_i = rowsum(dO_i * O_i)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  Strides s_q, s_k, s_v, s_o, s_do, s_dq, s_dk, s_dv;
  int H;
  int Sq, Skv;
  int nq, nk;  // query tiles per head (dQ kernel), key tiles per head (dK/dV kernel)
  int64_t BH;  // B * H
  int64_t hchunk_q, hchunk_k;  // heads per chunk of the causal orders (dQ, dK/dV kernels)
  TileMap map_q, map_k;        // workgroup -> (tile, b*H + h) of the dQ and dK/dV kernels
  Div31 dH;                    // division by H
  float c;     // scale * log2(e), kept >= FLT_MIN
  float scale;
};

// Launch geometry of the two backward kernels for head dim D.
struct BwdPlan {
  int dkdv_keys_per_workgroup;  // key tile of the dK/dV kernel
  int dkdv_query_step;          // queries per step of its loop
  int dq_queries_per_workgroup;  // query tile of the dQ kernel
  int dq_key_step;               // keys per step of its loop
  int threads_per_workgroup;
  int lds_bytes;                 // per workgroup, either kernel
};

BwdPlan bwd_plan(int D);

// Enqueue the dQ (and D_i) and dK/dV kernels on `stream` (p.nq, p.nk and the
// tile maps are filled in here).  D is 64, 128 or 256; the caller has validated everything.
hipError_t bwd_launch(BwdProblem p, int D, bool causal, int dtype, hipStream_t stream);

}  // namespace attn
