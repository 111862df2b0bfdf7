/*
 * Plain fp64 CPU oracle for exact attention:  O = softmax(scale * Q K^T) V,
 * plus the per-row log-sum-exp.  TEST INFRASTRUCTURE ONLY: the test-suite,
 * the smoke check and the benchmark's CPU-baseline leg call it; the GPU
 * library never does, and the two share no code.
 *
 * What it computes follows the three-step definition of standard attention
 * (zzszmyf.github.io notes "FlashAttention 原理是什么", section 2: S = QK^T,
 * P = softmax(S), O = PV; aiqz.cc Flash Attention IO article, section
 * 标准注意力瓶颈) with the max-subtracted row softmax of the cf-1.com
 * FlashAttention write-up, section 3.1 (m = max x, l = sum exp(x - m),
 * softmax = exp(x - m) / l).  Rows are handled one at a time, so no N x N
 * buffer is formed; nothing is tiled or merged online.
 *
 * Readings of what the pages leave open:
 *   - S is scaled by `scale` before the softmax (the pages' demo omits it).
 *   - grouped K/V heads: K and V carry Hkv heads, query head h reads K/V
 *     head h / (H / Hkv) (Hkv == H is ordinary multi-head attention).
 *   - causal: key j takes part in query row i iff j <= i + (Nk - Nq), i.e.
 *     the last query lines up with the last key (for Nq == Nk: j <= i); a
 *     masked key is excluded outright.  Causal calls need Nq <= Nk, so every
 *     row keeps at least key 0.
 *   - LSE_i = m_i + ln(l_i) over the scaled, masked scores (natural log).
 * Inputs are float32 arrays (bf16 data is widened exactly before the call);
 * every product and sum is carried in IEEE double, no fast-math.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One query row: flat row index r = (b*H + h)*Nq + i.  Writes d values of O
 * and one LSE.  `s` is a caller-provided scratch row of Nk doubles. */
static void oracle_row(const float* q, const float* k, const float* v,
                       int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                       double scale, int causal, int64_t r, double* s, double* o_row,
                       double* lse_out) {
  const int64_t bh = r / Nq;         /* (b*H + h) */
  const int64_t i = r % Nq;          /* query position inside the head */
  const int64_t b = bh / H, h = bh % H;
  const int64_t bkv = b * Hkv + h / (H / Hkv);   /* the K/V head it reads */
  const float* qi = q + r * d;
  const float* kh = k + bkv * Nk * d;
  const float* vh = v + bkv * Nk * d;
  /* keys j with j <= i + (Nk - Nq) when causal */
  const int64_t nkeys = causal ? (i + (Nk - Nq) + 1) : Nk;

  /* step 1: scores s_j = scale * <q_i, k_j> */
  double m = -INFINITY;
  for (int64_t j = 0; j < nkeys; ++j) {
    const float* kj = kh + j * d;
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += (double)qi[c] * (double)kj[c];
    s[j] = scale * dot;
    if (s[j] > m) m = s[j];
  }
  /* step 2: row softmax with the row max subtracted */
  double l = 0.0;
  for (int64_t j = 0; j < nkeys; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  /* step 3: O_i = sum_j p_j v_j / l */
  for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
  for (int64_t j = 0; j < nkeys; ++j) {
    const float* vj = vh + j * d;
    const double p = s[j];
    for (int64_t c = 0; c < d; ++c) o_row[c] += p * (double)vj[c];
  }
  for (int64_t c = 0; c < d; ++c) o_row[c] /= l;
  *lse_out = m + log(l);
}

/* Attention of q [B,H,Nq,d] over k, v [B,Hkv,Nk,d] for the query rows
 * listed in `rows` (flat indices into [B,H,Nq]); rows == NULL means every
 * row, in order.  O is [nrows, d], LSE [nrows].  Returns 0 on success, 1 on
 * a bad argument (including causal with Nq > Nk, or H not a multiple of
 * Hkv), 2 if scratch allocation fails. */
int oracle_attn_f64(const float* q, const float* k, const float* v,
                    int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                    double scale, int causal, const int64_t* rows, int64_t nrows,
                    double* O, double* LSE) {
  if (!q || !k || !v || !O || !LSE || B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1)
    return 1;
  if (H % Hkv != 0) return 1;
  if (causal && Nq > Nk) return 1;
  const int64_t total = B * H * Nq;
  if (!rows) nrows = total;
  if (nrows < 0) return 1;
  for (int64_t t = 0; t < nrows && rows; ++t)
    if (rows[t] < 0 || rows[t] >= total) return 1;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t t = 0; t < nrows; ++t) {
        const int64_t r = rows ? rows[t] : t;
        oracle_row(q, k, v, H, Hkv, Nq, Nk, d, scale, causal, r, s, O + t * d, LSE + t);
      }
      free(s);
    }
  }
  return failed ? 2 : 0;
}

/* Threads the OpenMP runtime will use for the next parallel region. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Backward pass.  For an upstream gradient dO of O, the gradients of the
 * attention above (square problem, Hkv == H, N queries and N keys) follow
 * from the chain rule through O = P V, P = row-softmax(S), S = scale Q K^T:
 *
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = <dO_i, v_j>
 *   dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')      (softmax Jacobian)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * with i, j over the visible pairs only (j <= i when causal).  These are
 * the quantities a recomputing backward pass rebuilds from Q, K, V and the
 * saved row statistics (zzszmyf.github.io notes, section 6; aiqz.cc
 * article, section 工程实现细节); the pages state that strategy, the formulas
 * are the chain rule.  A row pass over i gives dQ and each row's (m, l, D); a
 * key pass over j rebuilds P_ij from the same score expression and gives
 * dK and dV.  No N x N buffer is formed.
 * ---------------------------------------------------------------------- */

static double dot_f32(const float* a, const float* b, int64_t d) {
  double s = 0.0;
  for (int64_t c = 0; c < d; ++c) s += (double)a[c] * (double)b[c];
  return s;
}

/* Gradients for the heads listed in `heads` (flat b*H + h; NULL = every
 * head, in order).  dQ, dK, dV are [nheads, N, d].  Returns 0 on success,
 * 1 on a bad argument, 2 if scratch allocation fails. */
int oracle_attn_bwd_f64(const float* q, const float* k, const float* v, const float* dO,
                        int64_t B, int64_t H, int64_t N, int64_t d, double scale, int causal,
                        const int64_t* heads, int64_t nheads,
                        double* dQ, double* dK, double* dV) {
  if (!q || !k || !v || !dO || !dQ || !dK || !dV || B < 1 || H < 1 || N < 1 || d < 1)
    return 1;
  if (heads == NULL) nheads = B * H;
  if (nheads < 1) return 1;
  for (int64_t t = 0; t < nheads; ++t)
    if (heads && (heads[t] < 0 || heads[t] >= B * H)) return 1;
  double* m = (double*)malloc(sizeof(double) * (size_t)N);
  double* l = (double*)malloc(sizeof(double) * (size_t)N);
  double* D = (double*)malloc(sizeof(double) * (size_t)N);
  if (!m || !l || !D) {
    free(m); free(l); free(D);
    return 2;
  }
  int fail = 0;
  for (int64_t t = 0; t < nheads; ++t) {
    const int64_t bh = heads ? heads[t] : t;
    const float* qh = q + bh * N * d;
    const float* kh = k + bh * N * d;
    const float* vh = v + bh * N * d;
    const float* gh = dO + bh * N * d;
    double* dq = dQ + t * N * d;
    double* dk = dK + t * N * d;
    double* dv = dV + t * N * d;

    /* row pass: scores, softmax, dP, D_i = sum_j P_ij dP_ij, dS, dQ_i */
#pragma omp parallel
    {
      double* s = (double*)malloc(sizeof(double) * (size_t)N);
      double* gp = (double*)malloc(sizeof(double) * (size_t)N);
      if (!s || !gp) {
#pragma omp atomic write
        fail = 1;
      } else {
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < N; ++i) {
          const int64_t nk = causal ? i + 1 : N;
          double mx = -INFINITY;
          for (int64_t j = 0; j < nk; ++j) {
            s[j] = scale * dot_f32(qh + i * d, kh + j * d, d);
            if (s[j] > mx) mx = s[j];
          }
          double sum = 0.0;
          for (int64_t j = 0; j < nk; ++j) sum += exp(s[j] - mx);
          double Di = 0.0;
          for (int64_t j = 0; j < nk; ++j) {
            gp[j] = dot_f32(gh + i * d, vh + j * d, d);      /* dP_ij */
            Di += (exp(s[j] - mx) / sum) * gp[j];
          }
          m[i] = mx;
          l[i] = sum;
          D[i] = Di;
          for (int64_t c = 0; c < d; ++c) dq[i * d + c] = 0.0;
          for (int64_t j = 0; j < nk; ++j) {
            const double p = exp(s[j] - mx) / sum;
            const double ds = p * (gp[j] - Di);
            for (int64_t c = 0; c < d; ++c) dq[i * d + c] += ds * (double)kh[j * d + c];
          }
          for (int64_t c = 0; c < d; ++c) dq[i * d + c] *= scale;
        }
      }
      free(s);
      free(gp);
    }
    if (fail) break;

    /* key pass: P_ij rebuilt from the same scores, dV_j and dK_j */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < N; ++j) {
      for (int64_t c = 0; c < d; ++c) {
        dk[j * d + c] = 0.0;
        dv[j * d + c] = 0.0;
      }
      for (int64_t i = causal ? j : 0; i < N; ++i) {
        const double sij = scale * dot_f32(qh + i * d, kh + j * d, d);
        const double p = exp(sij - m[i]) / l[i];
        const double ds = p * (dot_f32(gh + i * d, vh + j * d, d) - D[i]);
        for (int64_t c = 0; c < d; ++c) {
          dv[j * d + c] += p * (double)gh[i * d + c];
          dk[j * d + c] += ds * (double)qh[i * d + c];
        }
      }
      for (int64_t c = 0; c < d; ++c) dk[j * d + c] *= scale;
    }
  }
  free(m);
  free(l);
  free(D);
  return fail ? 2 : 0;
}
