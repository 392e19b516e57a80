/*
 * attn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of the exact attention
 * forward, in float64.  Only tests/, the smoke check and the bench's CPU
 * baseline may load it; the product path never does.  It shares no code,
 * header, table or constant with the GPU library.
 *
 * What it computes (source: the docs.rs page "oxicuda-dnn 0.1.8,
 * src/attn/flash_attn/hopper.rs", doc comment of
 * FlashAttention3Plan::generate_forward, and the `causal` field of
 * FlashAttention3Config): for every batch b, head h and query row i,
 *
 *   A_i  = { j : 0 <= j < Skv, and j <= i + (Skv - Sq) when causal }
 *   s_ij = scale * sum_d q[b,h,i,d] * k[b,h,j,d]
 *   m_i  = max_{j in A_i} s_ij
 *   l_i  = sum_{j in A_i} exp(s_ij - m_i)
 *   O_i  = sum_{j in A_i} exp(s_ij - m_i) * v[b,h,j,:] / l_i
 *   LSE_i = m_i + ln(l_i)
 *
 * Readings where the page is silent: the log-sum-exp is the natural logarithm
 * of the scaled, masked scores; queries and keys may differ in length (the
 * page's kernel takes separate query and key/value lengths), and causal then
 * aligns the last query with the last key: query i (of Sq) keeps key j (of
 * Skv) iff j <= i + (Skv - Sq), which is j <= i when Sq == Skv; a query with
 * no key left (Sq > Skv) gets O = 0 and LSE = -inf; tensors are contiguous
 * Q, O [B,H,Sq,D], K, V [B,H,Skv,D], LSE [B,H,Sq]; inputs are the 16-bit
 * words the GPU receives (fp16 or bf16), widened exactly to float64.
 *
 * Three routines:
 *   oracle_attn_fwd        two passes per row (max, then sums), the definition
 *   oracle_attn_fwd_online keys in blocks with a running max m and running
 *                          sum l, rescaling the partial output when m grows
 *                          (the online softmax of the page's doc comment of
 *                          generate_forward); used to show tiling is exact
 *   oracle_attn_probs      the softmax matrix P itself, for small S
 * and, on float64 inputs, the same forward (oracle_attn_fwd_f64) and the
 * backward of the page's doc comment of generate_backward
 * (oracle_attn_bwd_f64; oracle_attn_bwd widens 16-bit inputs first).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double g_f16[65536];
static double g_bf16[65536];
static int g_tables_ready = 0;

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double mag;
  if (e == 0) {
    mag = ldexp((double)f, -24);
  } else if (e == 31) {
    mag = f ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(1024 + f), e - 25);
  }
  return sign ? -mag : mag;
}

/* bfloat16: the upper half of an IEEE binary32. */
static double decode_bf16(uint16_t h) {
  uint32_t w = (uint32_t)h << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static void init_tables(void) {
  if (g_tables_ready) return;
  for (int i = 0; i < 65536; ++i) {
    g_f16[i] = decode_f16((uint16_t)i);
    g_bf16[i] = decode_bf16((uint16_t)i);
  }
  g_tables_ready = 1;
}

static const double* table_for(int dtype) {
  return dtype == 0 ? g_f16 : g_bf16;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_decode(const uint16_t* bits, int dtype, int64_t n, double* out) {
  init_tables();
  const double* t = table_for(dtype);
  for (int64_t i = 0; i < n; ++i) out[i] = t[bits[i]];
}

/* Number of keys query i may attend to (keys 0 .. n-1). */
static int64_t allowed_keys(int64_t i, int64_t Sq, int64_t Skv, int causal) {
  if (!causal) return Skv;
  int64_t n = i + 1 + (Skv - Sq);
  return n < 0 ? 0 : (n < Skv ? n : Skv);
}

static void scores_row(const double* tab, const uint16_t* q, const uint16_t* k,
                       int64_t bh, int64_t i, int64_t Sq, int64_t Skv, int64_t D,
                       double scale, int64_t n, double* qd, double* s) {
  const uint16_t* qrow = q + (bh * Sq + i) * D;
  for (int64_t d = 0; d < D; ++d) qd[d] = tab[qrow[d]];
  for (int64_t j = 0; j < n; ++j) {
    const uint16_t* krow = k + (bh * Skv + j) * D;
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += qd[d] * tab[krow[d]];
    s[j] = scale * acc;
  }
}

/*
 * Queries of length Sq against keys/values of length Skv.  rows: flat query
 * row indices r = (b*H + h)*Sq + i, or NULL for all B*H*Sq rows in order.
 * o receives nrows*D values, lse nrows values.  Returns 0, or -1 when
 * scratch memory cannot be had.
 */
int oracle_attn_fwd_qk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                       int64_t D, double scale, int causal, const int64_t* rows,
                       int64_t nrows, double* o, double* lse) {
  init_tables();
  const double* tab = table_for(dtype);
  if (rows == NULL) nrows = B * H * Sq;
  int failed = 0;
#pragma omp parallel
  {
    double* qd = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
    double* s = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
    if (!qd || !s || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 8)
      for (int64_t t = 0; t < nrows; ++t) {
        int64_t r = rows ? rows[t] : t;
        int64_t bh = r / Sq, i = r % Sq;
        int64_t n = allowed_keys(i, Sq, Skv, causal);
        double* orow = o + t * D;
        if (n <= 0) {
          for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
          lse[t] = -INFINITY;
          continue;
        }
        scores_row(tab, q, k, bh, i, Sq, Skv, D, scale, n, qd, s);
        /* pass 1: the row maximum */
        double m = s[0];
        for (int64_t j = 1; j < n; ++j) m = s[j] > m ? s[j] : m;
        /* pass 2: normaliser and weighted sum of values */
        double l = 0.0;
        for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
        for (int64_t j = 0; j < n; ++j) {
          double p = exp(s[j] - m);
          l += p;
          const uint16_t* vrow = v + (bh * Skv + j) * D;
          for (int64_t d = 0; d < D; ++d) acc[d] += p * tab[vrow[d]];
        }
        for (int64_t d = 0; d < D; ++d) orow[d] = acc[d] / l;
        lse[t] = m + log(l);
      }
    }
    free(qd);
    free(s);
    free(acc);
  }
  return failed ? -1 : 0;
}

/* Equal query and key lengths S. */
int oracle_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                    double scale, int causal, const int64_t* rows,
                    int64_t nrows, double* o, double* lse) {
  return oracle_attn_fwd_qk(q, k, v, dtype, B, H, S, S, D, scale, causal, rows, nrows, o, lse);
}

/*
 * The same result reached blockwise: keys are visited in blocks of `block`,
 * keeping a running max m, a running sum l and an unnormalised output that is
 * rescaled by exp(m_old - m_new) whenever the max grows.  All rows.
 */
int oracle_attn_fwd_online(const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, int dtype, int64_t B, int64_t H,
                           int64_t S, int64_t D, double scale, int causal,
                           int64_t block, double* o, double* lse) {
  init_tables();
  if (block <= 0) return -1;
  const double* tab = table_for(dtype);
  int64_t nrows = B * H * S;
  int failed = 0;
#pragma omp parallel
  {
    double* qd = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
    double* s = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
    if (!qd || !s || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 8)
      for (int64_t r = 0; r < nrows; ++r) {
        int64_t bh = r / S, i = r % S;
        int64_t n = allowed_keys(i, S, S, causal);
        double* orow = o + r * D;
        scores_row(tab, q, k, bh, i, S, S, D, scale, n, qd, s);
        double m = -INFINITY, l = 0.0;
        for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
        for (int64_t j0 = 0; j0 < n; j0 += block) {
          int64_t j1 = j0 + block < n ? j0 + block : n;
          double mb = -INFINITY;
          for (int64_t j = j0; j < j1; ++j) mb = s[j] > mb ? s[j] : mb;
          double m_new = mb > m ? mb : m;
          double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
          l *= alpha;
          for (int64_t d = 0; d < D; ++d) acc[d] *= alpha;
          for (int64_t j = j0; j < j1; ++j) {
            double p = exp(s[j] - m_new);
            l += p;
            const uint16_t* vrow = v + (bh * S + j) * D;
            for (int64_t d = 0; d < D; ++d) acc[d] += p * tab[vrow[d]];
          }
          m = m_new;
        }
        if (n <= 0) {
          for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
          lse[r] = -INFINITY;
        } else {
          for (int64_t d = 0; d < D; ++d) orow[d] = acc[d] / l;
          lse[r] = m + log(l);
        }
      }
    }
    free(qd);
    free(s);
    free(acc);
  }
  return failed ? -1 : 0;
}

/* The softmax matrix P [B,H,S,S] (zero where masked), for small S. */
int oracle_attn_probs(const uint16_t* q, const uint16_t* k, int dtype,
                      int64_t B, int64_t H, int64_t S, int64_t D, double scale,
                      int causal, double* p) {
  init_tables();
  const double* tab = table_for(dtype);
  double* qd = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
  double* s = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
  if (!qd || !s) {
    free(qd);
    free(s);
    return -1;
  }
  for (int64_t bh = 0; bh < B * H; ++bh) {
    for (int64_t i = 0; i < S; ++i) {
      double* prow = p + (bh * S + i) * S;
      int64_t n = allowed_keys(i, S, S, causal);
      for (int64_t j = 0; j < S; ++j) prow[j] = 0.0;
      if (n <= 0) continue;
      scores_row(tab, q, k, bh, i, S, S, D, scale, n, qd, s);
      double m = s[0];
      for (int64_t j = 1; j < n; ++j) m = s[j] > m ? s[j] : m;
      double l = 0.0;
      for (int64_t j = 0; j < n; ++j) l += exp(s[j] - m);
      for (int64_t j = 0; j < n; ++j) prow[j] = exp(s[j] - m) / l;
    }
  }
  free(qd);
  free(s);
  return 0;
}

/*
 * ---------------------------------------------------------------------------
 * Float64 inputs.  The same forward definition on float64 arrays (contiguous
 * Q [B,H,Sq,D], K, V [B,H,Skv,D]), so that the backward below can be checked
 * by finite differences of it, and the backward itself.
 * ---------------------------------------------------------------------------
 */
static void scores_row_f64(const double* q, const double* k, int64_t bh, int64_t i,
                           int64_t Sq, int64_t Skv, int64_t D, double scale, int64_t n,
                           double* s) {
  const double* qrow = q + (bh * Sq + i) * D;
  for (int64_t j = 0; j < n; ++j) {
    const double* krow = k + (bh * Skv + j) * D;
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += qrow[d] * krow[d];
    s[j] = scale * acc;
  }
}

/* P_ij = exp(s_ij - m_i) / l_i over the n kept keys; returns LSE_i. */
static double softmax_row(double* s, int64_t n) {
  double m = s[0];
  for (int64_t j = 1; j < n; ++j) m = s[j] > m ? s[j] : m;
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) l += exp(s[j] - m);
  for (int64_t j = 0; j < n; ++j) s[j] = exp(s[j] - m) / l;
  return m + log(l);
}

int oracle_attn_fwd_f64(const double* q, const double* k, const double* v, int64_t B,
                        int64_t H, int64_t Sq, int64_t Skv, int64_t D, double scale,
                        int causal, double* o, double* lse) {
  int failed = 0;
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
    if (!p) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 8)
      for (int64_t r = 0; r < B * H * Sq; ++r) {
        const int64_t bh = r / Sq, i = r % Sq;
        const int64_t n = allowed_keys(i, Sq, Skv, causal);
        double* orow = o + r * D;
        for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
        if (n <= 0) {
          lse[r] = -INFINITY;
          continue;
        }
        scores_row_f64(q, k, bh, i, Sq, Skv, D, scale, n, p);
        lse[r] = softmax_row(p, n);
        for (int64_t j = 0; j < n; ++j) {
          const double* vrow = v + (bh * Skv + j) * D;
          for (int64_t d = 0; d < D; ++d) orow[d] += p[j] * vrow[d];
        }
      }
    }
    free(p);
  }
  return failed ? -1 : 0;
}

/*
 * The backward (source: the same page, doc comment of
 * FlashAttention3Plan::generate_backward): given the gradient dO of the
 * loss with respect to O, with P recomputed from the scores,
 *
 *   P_ij  = exp(s_ij - LSE_i) for j in A_i, 0 otherwise
 *   dV_j  = sum_i P_ij dO_i                 (dV = P^T dO)
 *   dP_ij = dO_i . v_j                      (dP = dO V^T)
 *   D_i   = sum_j dP_ij P_ij                (the page's rowsum(dP * P))
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j         (dQ = dS K)
 *   dK_j  = scale * sum_i dS_ij q_i         (dK = dS^T Q)
 *
 * dS is the gradient with respect to the scaled scores s = scale * q.k, so
 * the chain rule puts the factor `scale` on dQ and dK (the page lists
 * sm_scale among the kernel's parameters and leaves it out of the formulas).
 * A query with no key has P = 0: dQ_i = 0, D_i = 0.  delta receives D_i
 * [B,H,Sq]; dq [B,H,Sq,D], dk and dv [B,H,Skv,D].
 *
 * Two passes, each over independent outputs (so the result does not depend
 * on the thread count):
 *   1. per query row i: P_i. from the scores, LSE_i, dP_i., D_i, dS_i., dQ_i;
 *   2. per key row j: for every query i that keeps key j, P_ij recomputed as
 *      exp(s_ij - LSE_i) (the page's recomputation from the saved
 *      log-sum-exp), dP_ij and dS_ij as above, summed into dK_j and dV_j.
 * Returns 0, or -1 when scratch memory cannot be had.
 */
int oracle_attn_bwd_f64(const double* q, const double* k, const double* v, const double* dO,
                        int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                        double scale, int causal, double* dq, double* dk, double* dv,
                        double* delta) {
  int failed = 0;
  double* lse = (double*)malloc(sizeof(double) * (size_t)(B * H * Sq > 0 ? B * H * Sq : 1));
  if (!lse) return -1;
  /* pass 1: rows of dQ, D_i and LSE_i */
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
    double* ds = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
    if (!p || !ds) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < B * H * Sq; ++r) {
        const int64_t bh = r / Sq, i = r % Sq;
        const double* dorow = dO + r * D;
        double* dqrow = dq + r * D;
        for (int64_t d = 0; d < D; ++d) dqrow[d] = 0.0;
        const int64_t n = allowed_keys(i, Sq, Skv, causal);
        if (n <= 0) {
          delta[r] = 0.0;
          lse[r] = -INFINITY;
          continue;
        }
        scores_row_f64(q, k, bh, i, Sq, Skv, D, scale, n, p);
        lse[r] = softmax_row(p, n);
        /* dP_ij, then D_i = sum_j dP_ij P_ij */
        double di = 0.0;
        for (int64_t j = 0; j < n; ++j) {
          const double* vrow = v + (bh * Skv + j) * D;
          double dp = 0.0;
          for (int64_t d = 0; d < D; ++d) dp += dorow[d] * vrow[d];
          ds[j] = dp;
          di += dp * p[j];
        }
        delta[r] = di;
        for (int64_t j = 0; j < n; ++j) {
          const double dsj = p[j] * (ds[j] - di);
          const double* krow = k + (bh * Skv + j) * D;
          for (int64_t d = 0; d < D; ++d) dqrow[d] += scale * dsj * krow[d];
        }
      }
    }
    free(p);
    free(ds);
  }
  /* pass 2: rows of dK and dV */
  if (!failed) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t c = 0; c < B * H * Skv; ++c) {
      const int64_t bh = c / Skv, j = c % Skv;
      const double* krow = k + c * D;
      const double* vrow = v + c * D;
      double* dkrow = dk + c * D;
      double* dvrow = dv + c * D;
      for (int64_t d = 0; d < D; ++d) dkrow[d] = dvrow[d] = 0.0;
      for (int64_t i = 0; i < Sq; ++i) {
        if (j >= allowed_keys(i, Sq, Skv, causal)) continue;
        const int64_t r = bh * Sq + i;
        const double* qrow = q + r * D;
        const double* dorow = dO + r * D;
        double s = 0.0, dp = 0.0;
        for (int64_t d = 0; d < D; ++d) {
          s += qrow[d] * krow[d];
          dp += dorow[d] * vrow[d];
        }
        const double pij = exp(scale * s - lse[r]);
        const double dsij = pij * (dp - delta[r]);
        for (int64_t d = 0; d < D; ++d) {
          dkrow[d] += scale * dsij * qrow[d];
          dvrow[d] += pij * dorow[d];
        }
      }
    }
  }
  free(lse);
  return failed ? -1 : 0;
}

/* The backward of 16-bit inputs (widened exactly to float64 first). */
int oracle_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const uint16_t* dO, int dtype, int64_t B, int64_t H, int64_t Sq,
                    int64_t Skv, int64_t D, double scale, int causal, double* dq,
                    double* dk, double* dv, double* delta) {
  const int64_t nq = B * H * Sq * D, nk = B * H * Skv * D;
  double* qd = (double*)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1));
  double* dod = (double*)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1));
  double* kd = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
  double* vd = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
  int rc = -1;
  if (qd && dod && kd && vd) {
    oracle_decode(q, dtype, nq, qd);
    oracle_decode(dO, dtype, nq, dod);
    oracle_decode(k, dtype, nk, kd);
    oracle_decode(v, dtype, nk, vd);
    rc = oracle_attn_bwd_f64(qd, kd, vd, dod, B, H, Sq, Skv, D, scale, causal, dq, dk, dv,
                             delta);
  }
  free(qd);
  free(dod);
  free(kd);
  free(vd);
  return rc;
}

/*
 * dQ_i and D_i of sampled query rows only (rows: flat indices (b*H + h)*Sq + i),
 * the first pass of oracle_attn_bwd_f64 restricted to those rows: each needs
 * only its own row of scores, so it runs at any length.  16-bit inputs.
 * dq receives nrows*D values, delta nrows.  Returns 0, or -1 when scratch
 * memory cannot be had.
 */
int oracle_attn_bwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, int dtype, int64_t B, int64_t H, int64_t Sq,
                         int64_t Skv, int64_t D, double scale, int causal,
                         const int64_t* rows, int64_t nrows, double* dq, double* delta) {
  init_tables();
  const double* tab = table_for(dtype);
  (void)B;
  (void)H;
  int failed = 0;
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
    double* qd = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
    double* dod = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
    if (!p || !dp || !qd || !dod) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t t = 0; t < nrows; ++t) {
        const int64_t r = rows[t], bh = r / Sq, i = r % Sq;
        double* dqrow = dq + t * D;
        for (int64_t d = 0; d < D; ++d) {
          dqrow[d] = 0.0;
          qd[d] = tab[q[r * D + d]];
          dod[d] = tab[dO[r * D + d]];
        }
        const int64_t n = allowed_keys(i, Sq, Skv, causal);
        if (n <= 0) {
          delta[t] = 0.0;
          continue;
        }
        for (int64_t j = 0; j < n; ++j) {
          const uint16_t* krow = k + (bh * Skv + j) * D;
          const uint16_t* vrow = v + (bh * Skv + j) * D;
          double s = 0.0, g = 0.0;
          for (int64_t d = 0; d < D; ++d) {
            s += qd[d] * tab[krow[d]];
            g += dod[d] * tab[vrow[d]];
          }
          p[j] = scale * s;
          dp[j] = g;
        }
        softmax_row(p, n);
        double di = 0.0;
        for (int64_t j = 0; j < n; ++j) di += dp[j] * p[j];
        delta[t] = di;
        for (int64_t j = 0; j < n; ++j) {
          const double dsj = p[j] * (dp[j] - di);
          const uint16_t* krow = k + (bh * Skv + j) * D;
          for (int64_t d = 0; d < D; ++d) dqrow[d] += scale * dsj * tab[krow[d]];
        }
      }
    }
    free(p);
    free(dp);
    free(qd);
    free(dod);
  }
  return failed ? -1 : 0;
}

/*
 * dK_j and dV_j of sampled keys only (keys: flat indices (b*H + h)*Skv + j):
 * for every query i that keeps key j, LSE_i and D_i from a full pass over
 * that query's row, then P_ij = exp(s_ij - LSE_i), dS_ij = P_ij (dP_ij - D_i),
 * dK_j += scale dS_ij q_i, dV_j += P_ij dO_i (the same definition as
 * oracle_attn_bwd_f64).  Cost: (queries keeping the key) x Skv x D per key,
 * small for the last keys of a long causal sequence.  16-bit inputs; dk, dv
 * receive nkeys*D values.  Returns 0, or -1 when scratch memory cannot be had.
 */
int oracle_attn_bwd_keys(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, int dtype, int64_t B, int64_t H, int64_t Sq,
                         int64_t Skv, int64_t D, double scale, int causal,
                         const int64_t* keys, int64_t nkeys, double* dk, double* dv) {
  init_tables();
  const double* tab = table_for(dtype);
  (void)B;
  (void)H;
  int failed = 0;
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
    if (!p || !dp) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t t = 0; t < nkeys; ++t) {
        const int64_t c = keys[t], bh = c / Skv, j = c % Skv;
        double* dkrow = dk + t * D;
        double* dvrow = dv + t * D;
        for (int64_t d = 0; d < D; ++d) dkrow[d] = dvrow[d] = 0.0;
        for (int64_t i = 0; i < Sq; ++i) {
          const int64_t n = allowed_keys(i, Sq, Skv, causal);
          if (j >= n) continue;
          const uint16_t* qrow = q + (bh * Sq + i) * D;
          const uint16_t* dorow = dO + (bh * Sq + i) * D;
          /* the query's whole row: scores, dP, LSE_i, D_i */
          for (int64_t jj = 0; jj < n; ++jj) {
            const uint16_t* krow = k + (bh * Skv + jj) * D;
            const uint16_t* vrow = v + (bh * Skv + jj) * D;
            double s = 0.0, g = 0.0;
            for (int64_t d = 0; d < D; ++d) {
              s += tab[qrow[d]] * tab[krow[d]];
              g += tab[dorow[d]] * tab[vrow[d]];
            }
            p[jj] = scale * s;
            dp[jj] = g;
          }
          const double sj = p[j];
          const double lse = softmax_row(p, n);
          double di = 0.0;
          for (int64_t jj = 0; jj < n; ++jj) di += dp[jj] * p[jj];
          const double pij = exp(sj - lse);
          const double dsij = pij * (dp[j] - di);
          for (int64_t d = 0; d < D; ++d) {
            dkrow[d] += scale * dsij * tab[qrow[d]];
            dvrow[d] += pij * tab[dorow[d]];
          }
        }
      }
    }
    free(p);
    free(dp);
  }
  return failed ? -1 : 0;
}
