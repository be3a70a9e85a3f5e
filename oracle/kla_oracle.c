/*
 * kla_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, fp64 CPU oracle of the Kaczmarz Linear Attention forward
 * pass.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library; the product path never does.  It shares no code,
 * header or constant with the HIP library.
 *
 * What it computes (paper "Kaczmarz Linear Attention", arXiv 2605.08587,
 * Algorithm 1 left panel "Tokenwise update (one head)", with the coefficient of
 * Eq. (3)), per (sequence, head), in the row-vector convention where the state
 * S is d_k x d_v and a key k_t is a 1 x d_k row:
 *
 *     a_t  = exp(g_t)                       decay; the blog "From Gated DeltaNet
 *                                            to Kaczmarz" s.2 writes alpha_t = exp(g_t)
 *     S~   = a_t S_{t-1}                    forget first               (Alg. 1, forget)
 *     e_t  = v_t - k_t S~                   residual                   (Alg. 1, residual)
 *     b_t  = eta_t / (||k_t||^2 + eps)      Kaczmarz step, Eq. (3)     (Alg. 1, step size)
 *     S_t  = S~ + b_t k_t^T e_t             rank-one projection write  (Alg. 1, write)
 *     o_t  = q_t S_t                        readout on the q given (no 1/||q||;
 *                                            normalising q is the caller's job)
 *
 * Variants (the pages' ablations and readout, selected by `mode` / `normq`):
 *   mode 0  b_t = eta_t / (||k_t||^2 + eps)           the method, Eq. (3)
 *   mode 1  b_t = eta_t                               the gated delta rule's learned
 *                                                     coefficient (s.2; Table 5 "without
 *                                                     normalization")
 *   mode 2  b_t = 1 / (||k_t||^2 + eps)               Table 5 "key-norm only"
 *   mode 3, 4, 5  the mode-0 coefficient times 1/t, 1/sqrt(t), 1/log(t + 1),
 *                 t the absolute 1-based position in the sequence (Appendix D,
 *                 "sequence factor"; the second factor is printed without its
 *                 root in the extracted text and read as 1/sqrt(t))
 *   normq   o_t = q_t S_t / ||q_t||_2 (s.3.3, Algorithm 1 readout), 0 for q_t = 0
 *   gdiag   diagonal gating (Appendix B.5, "Extension to diagonal gating"): the decay is
 *           Diag(alpha_t) with one log-decay g_t[i] per key channel i, so the forget step
 *           scales row i of the state by exp(g_t[i]); everything else, the coefficient
 *           included, is unchanged (the appendix keeps the Kaczmarz coefficient as is)
 *
 * Readings of points the pages leave open:
 *   - if ||k_t||^2 + eps == 0 the step is b_t = 0 (no write): the constraint
 *     0 = v_t cannot be met and the minimal-change state is S~ itself;
 *   - every dot product is summed in natural index order in double;
 *   - a sequence of length 0 leaves S_T = S0.
 *
 * Inputs are the exact stored values (bf16 or fp32) widened to double by the
 * caller, so the oracle sees bit-identical data to the device path.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One tokenwise step on one head's state S (dk x dv, row-major, d_v fastest) at
 * absolute position t (1-based).  g points to the token's log-decay: one value, or dk
 * values (one per state row) when gdiag.  r is caller scratch of length dv.  Writes o
 * (length dv) if o != NULL. */
static void kla_oracle_token(double *S, const double *q, const double *k,
                             const double *v, const double *g, double eta, double eps,
                             int dk, int dv, double *r, double *o, int mode,
                             int normq, double t, int gdiag) {
  /* S~ = a S, or Diag(a) S */
  for (int i = 0; i < dk; ++i) {
    const double a = exp(gdiag ? g[i] : g[0]);
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
  }
  /* e = v - k S~ */
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += k[i] * S[(size_t)i * dv + j];
    r[j] = v[j] - acc;
  }
  /* b = eta / (||k||^2 + eps), b = 0 when the denominator vanishes */
  double kk = 0.0;
  for (int i = 0; i < dk; ++i) kk += k[i] * k[i];
  const double den = kk + eps;
  double b;
  if (mode == 1) {
    b = eta;
  } else if (mode == 2) {
    b = (den == 0.0) ? 0.0 : 1.0 / den;
  } else {
    b = (den == 0.0) ? 0.0 : eta / den;
    if (mode == 3) b /= t;
    else if (mode == 4) b /= sqrt(t);
    else if (mode == 5) b /= log(t + 1.0);
  }
  /* S = S~ + b k^T e */
  for (int i = 0; i < dk; ++i) {
    const double bk = b * k[i];
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bk * r[j];
  }
  /* o = q S, or q S / ||q|| */
  if (o) {
    double scale = 1.0;
    if (normq) {
      double qq = 0.0;
      for (int i = 0; i < dk; ++i) qq += q[i] * q[i];
      scale = (qq == 0.0) ? 0.0 : 1.0 / sqrt(qq);
    }
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];
      o[j] = acc * scale;
    }
  }
}

/*
 * Prefill: run the recurrence over every token of every sequence.
 *   q, k   [n_tok, H, dk]      v, o [n_tok, H, dv]      g, eta [n_tok, H]
 *          (g [n_tok, H, dk] when gdiag)
 *   S0     [n_seq, H, dk, dv]  (NULL = zeros)          S_T   [n_seq, H, dk, dv]
 *   cu     [n_seq + 1] token offsets of the packed sequences (cu[0] = 0).
 *   nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int kla_oracle_prefill_v(const double *q, const double *k, const double *v,
                         const double *g, const double *eta, double eps,
                         const double *S0, const int64_t *cu, int n_seq, int H,
                         int dk, int dv, double *o, double *S_T, int nthreads,
                         int mode, int normq, const int64_t *pos_offset, int gdiag) {
  if (!q || !k || !v || !g || !eta || !cu || !o || !S_T) return -1;
  if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  const long pairs = (long)n_seq * H;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
  for (long p = 0; p < pairs; ++p) {
    const int n = (int)(p / H), h = (int)(p % H);
    double *S = S_T + (size_t)p * dk * dv;
    double *r = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!r) { failed = 1; continue; }
    if (S0)
      memcpy(S, S0 + (size_t)p * dk * dv, sizeof(double) * (size_t)dk * dv);
    else
      memset(S, 0, sizeof(double) * (size_t)dk * dv);
    const int64_t base = pos_offset ? pos_offset[n] : 0;
    for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
      const size_t th = (size_t)t * H + h;
      kla_oracle_token(S, q + th * dk, k + th * dk, v + th * dv,
                       gdiag ? g + th * dk : g + th, eta[th], eps, dk, dv, r,
                       o + th * dv, mode, normq, (double)(base + (t - cu[n]) + 1),
                       gdiag);
    }
    free(r);
  }
  return failed ? -1 : 0;
}

/* The method itself: mode 0, o_t = q_t S_t. */
int kla_oracle_prefill(const double *q, const double *k, const double *v,
                       const double *g, const double *eta, double eps,
                       const double *S0, const int64_t *cu, int n_seq, int H,
                       int dk, int dv, double *o, double *S_T, int nthreads) {
  return kla_oracle_prefill_v(q, k, v, g, eta, eps, S0, cu, n_seq, H, dk, dv, o,
                              S_T, nthreads, 0, 0, NULL, 0);
}

/*
 * Decode: one token per sequence, B sequences, state updated in S_new.
 *   q, k [B, H, dk]   v, o [B, H, dv]   g, eta [B, H]   S, S_new [B, H, dk, dv]
 *   (g [B, H, dk] when gdiag)
 * S_new may equal S.
 */
int kla_oracle_decode_v(const double *q, const double *k, const double *v,
                        const double *g, const double *eta, double eps,
                        const double *S, int B, int H, int dk, int dv, double *o,
                        double *S_new, int nthreads, int mode, int normq,
                        const int64_t *pos_offset, int gdiag) {
  if (!q || !k || !v || !g || !eta || !S || !o || !S_new) return -1;
  if (B < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  const long pairs = (long)B * H;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(static) reduction(| : failed)
  for (long p = 0; p < pairs; ++p) {
    double *Sp = S_new + (size_t)p * dk * dv;
    double *r = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!r) { failed = 1; continue; }
    if (Sp != S + (size_t)p * dk * dv)
      memcpy(Sp, S + (size_t)p * dk * dv, sizeof(double) * (size_t)dk * dv);
    const double t = (double)((pos_offset ? pos_offset[p / H] : 0) + 1);
    kla_oracle_token(Sp, q + (size_t)p * dk, k + (size_t)p * dk,
                     v + (size_t)p * dv, gdiag ? g + (size_t)p * dk : g + p, eta[p],
                     eps, dk, dv, r, o + (size_t)p * dv, mode, normq, t, gdiag);
    free(r);
  }
  return failed ? -1 : 0;
}

/* The method itself: mode 0, o_t = q_t S_t. */
int kla_oracle_decode(const double *q, const double *k, const double *v,
                      const double *g, const double *eta, double eps,
                      const double *S, int B, int H, int dk, int dv, double *o,
                      double *S_new, int nthreads) {
  return kla_oracle_decode_v(q, k, v, g, eta, eps, S, B, H, dk, dv, o, S_new,
                             nthreads, 0, 0, NULL, 0);
}

/* Threads the OpenMP runtime would use (for reporting the CPU baseline). */
int kla_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
