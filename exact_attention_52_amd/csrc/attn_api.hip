// attn_api.hip -- the C ABI declared in include/attn.h: argument checks,
// launch planning, device check and kernel dispatch for gfx950.
//
// The checks mirror the page's validate_config (docs.rs "oxicuda-dnn 0.1.8,
// src/attn/flash_attn/hopper.rs"): head_dim must be one of 64/128/256, the
// float type F16 or BF16; the launch follows its launch_params: one workgroup
// per (query tile, batch*head), ceil(S / block_m) query tiles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "attn.h"
#include "attn_bwd.hpp"
#include "attn_common.hpp"
#include "attn_fwd_kernel.hpp"
#include "attn_variants.hpp"

namespace {

// Per-head-dim tile shapes (TileCfg arguments: D, query waves, key waves,
// keys per tile, ping-pong kernel, staggered copies, K/V LDS stages,
// producer wave, in-wave pipeline).
//   D=64 : kernel 1, 4 query waves x 32 rows = 128 rows, 64-key tiles, two
//          K/V stages: 35 KiB of LDS and 114 VGPRs, so four workgroups share
//          a CU (four waves per SIMD).  Each one's copy waits, prologue and
//          output overlap the others' loops, and the waves on a SIMD belong
//          to different workgroups, so they do not meet at the same barriers
//          and fill each other's MFMA and VALU gaps.
//   D=128: ping-pong kernel, 8 waves = 256 rows, 128-key tiles, two stages,
//          133 KiB LDS
//   D=256: grids of at least 512 128-row tiles (use_inwave_256): the
//          in-wave pipelined kernel, 4 waves x 32 rows = 128 rows, 64-key
//          tiles, two stages, 133 KiB LDS, one wave per SIMD; smaller grids:
//          kernel 1 with staggered copies over two stages, 2 query waves = 64
//          rows (the page's 64-row Q tile for D=256), each 64-key tile split
//          over 2 key waves, 134.5 KiB LDS (with the key-split merge's row
//          sums)
using Cfg64 = attn::TileCfg<64, 4, 1, 64, false, false, 2>;
using Cfg128 = attn::TileCfg<128, 8, 1, 128, true>;
using Cfg256 = attn::TileCfg<256, 4, 1, 64, false, false, 2, false, true>;
using Cfg256Small = attn::TileCfg<256, 2, 2, 64, false, true>;

template <class C>
void fill_plan(int64_t B, int64_t H, int64_t S, attn_fwd_plan_t* p) {
  p->block_m = C::BM;
  p->block_n = C::BN;
  p->kv_stages = C::STAGES;
  p->waves_q = C::QW;
  p->waves_k = C::KW;
  p->threads_per_workgroup = C::NT;
  p->lds_bytes = C::LDS_BYTES;
  p->num_q_tiles = (S + C::BM - 1) / C::BM;
  p->num_workgroups = p->num_q_tiles * B * H;
}

int plan_for(int64_t B, int64_t H, int64_t S, int64_t D, attn_fwd_plan_t* p) {
  switch (D) {
    case 64: fill_plan<Cfg64>(B, H, S, p); break;
    case 128: fill_plan<Cfg128>(B, H, S, p); break;
    default:
      if (attn::use_inwave_256(B * H, S))
        fill_plan<Cfg256>(B, H, S, p);
      else
        fill_plan<Cfg256Small>(B, H, S, p);
      break;
  }
  if (p->num_workgroups > (int64_t)0x7FFFFFFF)
    return fail(ATTN_ERR_BAD_SHAPE, "grid of %lld workgroups exceeds the launch limit",
                (long long)p->num_workgroups);
  return ATTN_OK;
}

template <class C, bool CAUSAL, int DT>
int launch(const attn::Problem& pr, hipStream_t stream) {
  if constexpr (C::PINGPONG)
    hipLaunchKernelGGL((attn::attn_fwd_pingpong_kernel<C, CAUSAL, DT>), dim3((unsigned)pr.G), dim3(C::NT), 0,
                       stream, pr);
  else if constexpr (C::INWAVE)
    hipLaunchKernelGGL((attn::attn_fwd_inwave_kernel<C, CAUSAL, DT>), dim3((unsigned)pr.G), dim3(C::NT), 0, stream,
                       pr);
  else
    hipLaunchKernelGGL((attn::attn_fwd_kernel<C, CAUSAL, DT>), dim3((unsigned)pr.G), dim3(C::NT), 0, stream, pr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

template <class C>
int dispatch(const attn::Problem& pr, bool causal, int dtype, hipStream_t st) {
  if (dtype == ATTN_F16)
    return causal ? launch<C, true, attn::DT_F16>(pr, st) : launch<C, false, attn::DT_F16>(pr, st);
  return causal ? launch<C, true, attn::DT_BF16>(pr, st) : launch<C, false, attn::DT_BF16>(pr, st);
}

// One 4-D tensor [B,H,rows,D] with the last dimension contiguous.
struct View {
  const void* p;
  int64_t sb, sh, ss;  // elements
  int64_t rows;
  const char* name;
};

// Strides of dimensions of size <= 1 never address anything: normalise them
// so that the checks and the kernel see the contiguous value.
void normalise(View& t, int64_t B, int64_t H, int64_t D) {
  if (t.rows <= 1) t.ss = D;
  if (H <= 1) t.sh = 0;
  if (B <= 1) t.sb = 0;
}

int check_view(const View& t, int64_t B, int64_t H, int64_t D) {
  if (t.sb < 0 || t.sh < 0 || t.ss < 0)
    return fail(ATTN_ERR_BAD_ARGUMENT, "%s strides must be >= 0", t.name);
  if (t.ss < D)
    return fail(ATTN_ERR_BAD_ARGUMENT, "%s row stride %lld is shorter than a row (%lld)", t.name, (long long)t.ss,
                (long long)D);
  if ((t.sb | t.sh | t.ss) & 7)
    return fail(ATTN_ERR_MISALIGNED, "%s strides must be multiples of 8 elements (16 bytes)", t.name);
  // one head's rows are addressed with 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 30;
  if (t.ss > lim || (t.rows > 0 && (t.rows - 1) > (lim - D) / t.ss))
    return fail(ATTN_ERR_BAD_SHAPE, "%s: one head spans more than 2 GiB", t.name);
  // the whole tensor within int64
  const int64_t big = (int64_t)1 << 60;
  if ((B > 0 && t.sb > big / B) || (H > 0 && t.sh > big / H))
    return fail(ATTN_ERR_BAD_SHAPE, "%s strides overflow", t.name);
  return ATTN_OK;
}

// Bytes from the tensor's base pointer to one past its last element.
int64_t extent_bytes(const View& t, int64_t B, int64_t H, int64_t D) {
  if (B == 0 || H == 0 || t.rows == 0) return 0;
  return 2 * ((B - 1) * t.sb + (H - 1) * t.sh + (t.rows - 1) * t.ss + D);
}

// The output must not address one element twice: with the dimensions of
// size > 1 sorted by stride, each stride must step over the whole previous
// dimension.
bool self_disjoint(const View& t, int64_t B, int64_t H, int64_t D) {
  int64_t dims[4][2] = {{D, 1}, {t.rows, t.ss}, {H, t.sh}, {B, t.sb}};
  int n = 0;
  int64_t d[4][2];
  for (auto& x : dims)
    if (x[0] > 1) d[n][0] = x[0], d[n][1] = x[1], ++n;
  for (int i = 1; i < n; ++i)
    for (int j = i; j > 0 && d[j][1] < d[j - 1][1]; --j) std::swap(d[j], d[j - 1]);
  for (int i = 1; i < n; ++i)
    if (d[i][1] < d[i - 1][1] * d[i - 1][0]) return false;
  return true;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t Sq,
        int64_t Skv, int64_t D, View vq, View vk, View vv, View vo, float scale, int causal, int dtype,
        void* stream, int variant = 0) {
  if (B < 0 || H < 0 || Sq < 0 || Skv < 0)
    return fail(ATTN_ERR_BAD_SHAPE, "B, H, Sq and Skv must be >= 0 (got B=%lld H=%lld Sq=%lld Skv=%lld)",
                (long long)B, (long long)H, (long long)Sq, (long long)Skv);
  int st = check_sizes(B, H, Sq > Skv ? Sq : Skv, D, dtype);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale)) return fail(ATTN_ERR_BAD_SCALE, "scale must be finite (got %g)", (double)scale);
  if (B == 0 || H == 0 || Sq == 0) return ok();  // empty: nothing to compute
  // with no keys nothing is read from k or v, which may then be NULL
  if (!q || !o || !lse || (Skv > 0 && (!k || !v)))
    return fail(ATTN_ERR_NULL_PTR, "q, k, v, o and lse must be non-NULL");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15)
    return fail(ATTN_ERR_MISALIGNED, "q, k, v and o must be 16-byte aligned");
  if ((uintptr_t)lse & 3) return fail(ATTN_ERR_MISALIGNED, "lse must be 4-byte aligned");
  for (View* t : {&vq, &vk, &vv, &vo}) {
    normalise(*t, B, H, D);
    st = check_view(*t, B, H, D);
    if (st != ATTN_OK) return st;
  }
  if (!self_disjoint(vo, B, H, D)) return fail(ATTN_ERR_ALIASING, "o strides make rows overlap");
  const int64_t nq_ = extent_bytes(vq, B, H, D), nk = extent_bytes(vk, B, H, D), nv = extent_bytes(vv, B, H, D);
  const int64_t no = extent_bytes(vo, B, H, D), nl = B * H * Sq * 4;
  if (overlaps(o, no, q, nq_) || overlaps(o, no, k, nk) || overlaps(o, no, v, nv) || overlaps(o, no, lse, nl))
    return fail(ATTN_ERR_ALIASING, "o overlaps q, k, v or lse");
  if (overlaps(lse, nl, q, nq_) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nv))
    return fail(ATTN_ERR_ALIASING, "lse overlaps q, k or v");
  attn_fwd_plan_t plan;
  st = plan_for(B, H, Sq, D, &plan);
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;

  attn::Problem pr;
  pr.q = (const uint16_t*)q, pr.k = (const uint16_t*)k, pr.v = (const uint16_t*)v;
  pr.o = (uint16_t*)o, pr.lse = lse;
  pr.q_sb = vq.sb, pr.q_sh = vq.sh, pr.k_sb = vk.sb, pr.k_sh = vk.sh;
  pr.v_sb = vv.sb, pr.v_sh = vv.sh, pr.o_sb = vo.sb, pr.o_sh = vo.sh;
  pr.q_ss = (int)vq.ss, pr.k_ss = (int)vk.ss, pr.v_ss = (int)vv.ss, pr.o_ss = (int)vo.ss;
  pr.Sq = (int)Sq, pr.Skv = (int)Skv, pr.H = (int)H, pr.nq = (int)plan.num_q_tiles;
  pr.G = plan.num_workgroups;
  pr.hchunk = attn::causal_head_chunk(Skv, D);
  // |scale| * log2(e), kept >= FLT_MIN: a masked score (-inf) times c must
  // stay -inf, never NaN, and for scale == 0 every kept score times FLT_MIN
  // is far below one ulp of the row max, so the softmax is exactly uniform.
  // A negative scale multiplies -Q (sign flips in registers, exact) by |scale|.
  float c = (float)(std::fabs((double)scale) * 1.4426950408889634074);
  if (c < FLT_MIN) c = FLT_MIN;
  pr.c = c;
  pr.qsign = scale < 0.f ? 0x80008000u : 0u;
  hipStream_t hs = (hipStream_t)stream;
  const bool cz = causal != 0;
  pr.map = attn::make_tile_map(pr.G, pr.nq, cz, pr.hchunk);
  pr.dH = attn::make_div31((uint32_t)H);
  if (variant != 0) {
    pr.G = B * H;  // the variant sets its own tile count and grid from B*H
    const hipError_t e = attn::variant_launch(pr, (int)D, cz, dtype, variant, hs);
    if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "variant %d launch failed: %s", variant, hipGetErrorString(e));
    return ok();
  }
  switch (D) {
    case 64: return dispatch<Cfg64>(pr, cz, dtype, hs);
    case 128: return dispatch<Cfg128>(pr, cz, dtype, hs);
    default:
      return plan.block_m == Cfg256::BM ? dispatch<Cfg256>(pr, cz, dtype, hs)
                                        : dispatch<Cfg256Small>(pr, cz, dtype, hs);
  }
}

// Scratch of attn_bwd_noalloc: the backward's per-row D_i, in a file-scope
// device array so that the call allocates nothing.  Each GPU holds its own
// copy (16 MiB) from the library's load until the process ends; host code
// reaches it only through the address hipGetSymbolAddress returns for the
// current device, never through the array's name.
constexpr int64_t kNoAllocRows = (int64_t)1 << 22;
static __device__ __align__(256) float scratch[kNoAllocRows];

std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices];  // guarded by g_scratch_mutex

// This device's address of `scratch`, looked up once per device with the
// device current.
int scratch_address(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "no current HIP device (%s)", hipGetErrorString(e));
  if (dev >= kMaxDevices)
    return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "device %d beyond the %d the scratch table covers", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(ATTN_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

// The backward of attn_bwd_strided; with use_scratch (attn_bwd_noalloc) D_i
// goes to this device's copy of the file-scope scratch array instead of the
// caller's delta.
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
             void* dk, void* dv, float* delta, bool use_scratch, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
             int64_t D,
             const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides, const int64_t* o_strides,
             const int64_t* do_strides, const int64_t* dq_strides, const int64_t* dk_strides,
             const int64_t* dv_strides, float scale, int causal, int dtype, void* stream) {
  if (B < 0 || H < 0 || Sq < 0 || Skv < 0)
    return fail(ATTN_ERR_BAD_SHAPE, "B, H, Sq and Skv must be >= 0 (got B=%lld H=%lld Sq=%lld Skv=%lld)",
                (long long)B, (long long)H, (long long)Sq, (long long)Skv);
  int st = check_sizes(B, H, Sq > Skv ? Sq : Skv, D, dtype);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale)) return fail(ATTN_ERR_BAD_SCALE, "scale must be finite (got %g)", (double)scale);
  if (use_scratch && B * H * Sq > kNoAllocRows)
    return fail(ATTN_ERR_BAD_ARGUMENT,
                "B*H*Sq = %lld rows exceed the %lld rows of D_i the no-allocation scratch holds",
                (long long)(B * H * Sq), (long long)kNoAllocRows);
  if (B == 0 || H == 0 || (Sq == 0 && Skv == 0)) return ok();
  const bool has_q = Sq > 0, has_k = Skv > 0;
  if ((has_q && (!q || !o || !dO || !lse || !dq || (!use_scratch && !delta))) || (has_k && (!k || !v || !dk || !dv)))
    return fail(ATTN_ERR_NULL_PTR, use_scratch ? "q, k, v, o, lse, dO, dq, dk and dv must be non-NULL"
                                               : "q, k, v, o, lse, dO, dq, dk, dv and delta must be non-NULL");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dO | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) & 15)
    return fail(ATTN_ERR_MISALIGNED, "q, k, v, o, dO, dq, dk and dv must be 16-byte aligned");
  if (((uintptr_t)lse | (uintptr_t)delta) & 3) return fail(ATTN_ERR_MISALIGNED, "lse and delta must be 4-byte aligned");
  auto view = [&](const void* ptr, const int64_t* sts, int64_t rows, const char* name) {
    View t = {ptr, H * rows * D, rows * D, D, rows, name};
    if (sts) t.sb = sts[0], t.sh = sts[1], t.ss = sts[2];
    normalise(t, B, H, D);
    return t;
  };
  View vs[8] = {view(q, q_strides, Sq, "q"),    view(k, k_strides, Skv, "k"),   view(v, v_strides, Skv, "v"),
                view(o, o_strides, Sq, "o"),    view(dO, do_strides, Sq, "dO"), view(dq, dq_strides, Sq, "dq"),
                view(dk, dk_strides, Skv, "dk"), view(dv, dv_strides, Skv, "dv")};
  for (const View& t : vs) {
    if (t.rows == 0) continue;
    st = check_view(t, B, H, D);
    if (st != ATTN_OK) return st;
  }
  for (int i = 5; i < 8; ++i)
    if (vs[i].rows > 0 && !self_disjoint(vs[i], B, H, D))
      return fail(ATTN_ERR_ALIASING, "%s strides make rows overlap", vs[i].name);
  const int64_t nr = B * H * Sq * 4;
  struct Buf {
    const void* p;
    int64_t n;
  };
  // the scratch is the library's own memory: no caller buffer can overlap it
  const Buf outs[4] = {{dq, extent_bytes(vs[5], B, H, D)},
                       {dk, extent_bytes(vs[6], B, H, D)},
                       {dv, extent_bytes(vs[7], B, H, D)},
                       {delta, use_scratch ? 0 : nr}};
  const Buf ins[6] = {{q, extent_bytes(vs[0], B, H, D)}, {k, extent_bytes(vs[1], B, H, D)},
                      {v, extent_bytes(vs[2], B, H, D)}, {o, extent_bytes(vs[3], B, H, D)},
                      {dO, extent_bytes(vs[4], B, H, D)}, {lse, nr}};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(ATTN_ERR_ALIASING, "dq, dk, dv and delta must not overlap each other");
    for (const Buf& b : ins)
      if (overlaps(outs[i].p, outs[i].n, b.p, b.n))
        return fail(ATTN_ERR_ALIASING, "dq, dk, dv and delta must not overlap q, k, v, o, dO or lse");
  }
  const attn::BwdPlan plan = attn::bwd_plan((int)D);
  const int64_t gq = B * H * ((Sq + plan.dq_queries_per_workgroup - 1) / plan.dq_queries_per_workgroup);
  const int64_t gk = B * H * ((Skv + plan.dkdv_keys_per_workgroup - 1) / plan.dkdv_keys_per_workgroup);
  if (gq > 0x7FFFFFFF || gk > 0x7FFFFFFF)
    return fail(ATTN_ERR_BAD_SHAPE, "grid exceeds the launch limit");
  st = check_device();
  if (st != ATTN_OK) return st;
  if (use_scratch && Sq > 0) {
    st = scratch_address(&delta);
    if (st != ATTN_OK) return st;
  }

  attn::BwdProblem p;
  p.q = (const uint16_t*)q, p.k = (const uint16_t*)k, p.v = (const uint16_t*)v, p.o = (const uint16_t*)o;
  p.dO = (const uint16_t*)dO, p.lse = lse, p.delta = delta;
  p.dq = (uint16_t*)dq, p.dk = (uint16_t*)dk, p.dv = (uint16_t*)dv;
  attn::Strides* ps[8] = {&p.s_q, &p.s_k, &p.s_v, &p.s_o, &p.s_do, &p.s_dq, &p.s_dk, &p.s_dv};
  for (int i = 0; i < 8; ++i) *ps[i] = attn::Strides{vs[i].sb, vs[i].sh, (int)vs[i].ss};
  p.H = (int)H;
  p.Sq = (int)Sq, p.Skv = (int)Skv, p.nq = 0, p.nk = 0, p.BH = B * H;
  // the dQ kernel streams K and V of its head, the dK/dV kernel Q and dO
  p.hchunk_q = attn::causal_head_chunk(Skv, D);
  p.hchunk_k = attn::causal_head_chunk(Sq, D);
  p.dH = attn::make_div31((uint32_t)H);
  // the backward masks P itself (never a score), so c may take any sign;
  // a tiny positive c is kept >= FLT_MIN as in the forward
  float c = (float)((double)scale * 1.4426950408889634074);
  p.c = (c >= 0.f && c < FLT_MIN) ? FLT_MIN : c;
  p.scale = scale;
  const hipError_t e = attn::bwd_launch(p, (int)D, causal != 0, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
             int64_t S, int64_t D, float scale, int causal, int dtype, void* stream) {
  // contiguous [B,H,S,D]; the sizes are checked before any stride is formed
  const int st = check_sizes(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  const int64_t sh = S * D, sb = H * S * D;
  const View packed = {nullptr, sb, sh, D, S, "q"};
  View vq = packed, vk = packed, vv = packed, vo = packed;
  vk.name = "k", vv.name = "v", vo.name = "o";
  return run(q, k, v, o, lse, B, H, S, S, D, vq, vk, vv, vo, scale, causal, dtype, stream);
}

int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t S, int64_t D, float scale, int causal, int dtype, int variant, void* stream) {
  const int st = check_sizes(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  const int vbm = variant > 0 && variant < attn::kNumVariants ? attn::variant_block_m((int)D, variant, B * H, S) : 0;
  if (variant < 0 || variant >= attn::kNumVariants || (variant > 0 && vbm == 0))
    return fail(ATTN_ERR_BAD_ARGUMENT, "variant %d not available for head_dim %lld (0..%d for D 64 and 128; 0, 5, 6 for 256)",
                variant, (long long)D, attn::kNumVariants - 1);
  if (variant > 0 && B * H * ((S + vbm - 1) / vbm) >
                         0x7FFFFFFF)
    return fail(ATTN_ERR_BAD_SHAPE, "grid exceeds the launch limit");
  const int64_t sh = S * D, sb = H * S * D;
  const View packed = {nullptr, sb, sh, D, S, "q"};
  View vq = packed, vk = packed, vv = packed, vo = packed;
  vk.name = "k", vv.name = "v", vo.name = "o";
  return run(q, k, v, o, lse, B, H, S, S, D, vq, vk, vv, vo, scale, causal, dtype, stream, variant);
}

int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t Sq, int64_t Skv, int64_t D, const int64_t* q_strides, const int64_t* k_strides,
                     const int64_t* v_strides, const int64_t* o_strides, float scale, int causal, int dtype,
                     void* stream) {
  // NULL strides mean contiguous [B,H,rows,D]; the sizes are checked before
  // any stride is formed
  if (Sq < 0 || Skv < 0)
    return fail(ATTN_ERR_BAD_SHAPE, "Sq and Skv must be >= 0 (got Sq=%lld Skv=%lld)", (long long)Sq,
                (long long)Skv);
  const int st0 = check_sizes(B, H, Sq > Skv ? Sq : Skv, D, dtype);
  if (st0 != ATTN_OK) return st0;
  auto view = [&](const int64_t* st, int64_t rows, const char* name) {
    View t = {nullptr, H * rows * D, rows * D, D, rows, name};
    if (st) t.sb = st[0], t.sh = st[1], t.ss = st[2];
    return t;
  };
  return run(q, k, v, o, lse, B, H, Sq, Skv, D, view(q_strides, Sq, "q"), view(k_strides, Skv, "k"),
             view(v_strides, Skv, "v"), view(o_strides, Sq, "o"), scale, causal, dtype, stream);
}

int attn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                     void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                     int64_t D, const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                     const int64_t* o_strides, const int64_t* do_strides, const int64_t* dq_strides,
                     const int64_t* dk_strides, const int64_t* dv_strides, float scale, int causal, int dtype,
                     void* stream) {
  return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, delta, false, B, H, Sq, Skv, D, q_strides, k_strides, v_strides,
                  o_strides, do_strides, dq_strides, dk_strides, dv_strides, scale, causal, dtype, stream);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                     void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                     float scale, int causal, int dtype, void* stream) {
  return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, nullptr, true, B, H, Sq, Skv, D, nullptr, nullptr, nullptr, nullptr,
                  nullptr, nullptr, nullptr, nullptr, scale, causal, dtype, stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
             void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
             int64_t D, float scale, int causal, int dtype, void* stream) {
  // contiguous tensors: the strided entry with every stride array NULL
  return attn_bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, Sq, Skv, D, nullptr, nullptr, nullptr,
                          nullptr, nullptr, nullptr, nullptr, nullptr, scale, causal, dtype, stream);
}

int attn_fwd_plan(int64_t B, int64_t H, int64_t S, int64_t D, int causal, int dtype, attn_fwd_plan_t* out) {
  (void)causal;
  if (!out) return fail(ATTN_ERR_NULL_PTR, "out must be non-NULL");
  int st = check_sizes(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  st = plan_for(B, H, S, D, out);
  if (st != ATTN_OK) return st;
  return ok();
}

int attn_fwd_workgroup_tile(int64_t B, int64_t H, int64_t S, int64_t D, int causal, int dtype, int64_t wg,
                            int64_t* q_tile, int64_t* bh) {
  if (!q_tile || !bh) return fail(ATTN_ERR_NULL_PTR, "q_tile and bh must be non-NULL");
  attn_fwd_plan_t p;
  int st = attn_fwd_plan(B, H, S, D, causal, dtype, &p);
  if (st != ATTN_OK) return st;
  if (wg < 0 || wg >= p.num_workgroups)
    return fail(ATTN_ERR_BAD_ARGUMENT, "workgroup %lld outside [0, %lld)", (long long)wg,
                (long long)p.num_workgroups);
  const attn::TileMap m = attn::make_tile_map(p.num_workgroups, p.num_q_tiles, causal != 0, attn::causal_head_chunk(S, D));
  uint32_t t = 0, b = 0;
  if (causal)
    attn::workgroup_tile<true>(m, (uint32_t)wg, &t, &b);
  else
    attn::workgroup_tile<false>(m, (uint32_t)wg, &t, &b);
  *q_tile = t;
  *bh = b;
  return ok();
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL_PTR: return "null pointer";
    case ATTN_ERR_BAD_SHAPE: return "bad shape";
    case ATTN_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head dim";
    case ATTN_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case ATTN_ERR_MISALIGNED: return "misaligned pointer";
    case ATTN_ERR_BAD_SCALE: return "bad scale";
    case ATTN_ERR_ALIASING: return "aliasing buffers";
    case ATTN_ERR_UNSUPPORTED_DEVICE: return "unsupported device";
    case ATTN_ERR_LAUNCH: return "launch failed";
    case ATTN_ERR_BAD_ARGUMENT: return "bad argument";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
