/*
 * Oracle for the gated delta rule — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check in __graft_entry__.py and the CPU-baseline leg of
 * bench.py may load this library.  The product path (libgdn) never links or calls it,
 * and the two share no code.
 *
 * What it computes (plain definition, fp64, token by token).  For every sequence n and
 * every value head h, with key/query head hk = h / (H / Hg) (contiguous grouping, as
 * the MegaGDN-PTO page states for GQA in its "Python interface" part, section 5.2):
 *
 *     S   <- h0[n, h]^T                              (S is Dv x Dk; zero when h0 is NULL)
 *     for each token t of the sequence, in order:
 *         S   <- exp(g_t) * S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *         o_t <- scale * S q_t                       (uses the state after token t)
 *     ht[n, h] <- S^T                                (Dk x Dv, the [B,H,K,V] state layout
 *                                                     given in the FlashQLA how-to, step 5.3)
 *
 * This is the gated delta-rule recurrence whose chunked evaluation the MegaGDN-PTO page
 * describes in section 1.1 (the seven-stage pipeline); the chunked form reaches the same
 * result up to rounding order.  The product S (I - beta k k^T) is expanded by
 * distributivity as S - beta (S k) k^T, which keeps the cost at O(Dk*Dv) per token.
 *
 * Layouts (all contiguous, row-major, token axis packed over sequences):
 *   q, k   [Ttot, Hg, Dk]     v, o  [Ttot, H, Dv]     g, beta [Ttot, H]
 *   h0, ht [N, H, Dk, Dv]
 * Sequence n occupies tokens start[n] .. start[n] + len[n] - 1.
 * pairs: optional list of (n * H + h) indices to evaluate (NULL = all pairs); outputs of
 * pairs not listed are left untouched.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void run_pair(int64_t start, int64_t len, int32_t h, int32_t H, int32_t Hg,
                     int32_t Dk, int32_t Dv, const double* q, const double* k,
                     const double* v, const double* g, const double* beta,
                     const double* h0_nh, double scale, double* o, double* ht_nh,
                     double* S, double* Sk) {
  const int32_t group = H / Hg;
  const int32_t hk = h / group;

  /* S = h0^T, or zero. */
  for (int32_t i = 0; i < Dv; ++i)
    for (int32_t j = 0; j < Dk; ++j)
      S[(int64_t)i * Dk + j] = h0_nh ? h0_nh[(int64_t)j * Dv + i] : 0.0;

  for (int64_t t = start; t < start + len; ++t) {
    const double* kt = k + (t * Hg + hk) * (int64_t)Dk;
    const double* qt = q + (t * Hg + hk) * (int64_t)Dk;
    const double* vt = v + (t * H + h) * (int64_t)Dv;
    const double decay = exp(g[t * H + h]);
    const double b = beta[t * H + h];

    /* Sk = S k_t */
    for (int32_t i = 0; i < Dv; ++i) {
      double acc = 0.0;
      for (int32_t j = 0; j < Dk; ++j) acc += S[(int64_t)i * Dk + j] * kt[j];
      Sk[i] = acc;
    }
    /* S = decay * (S - b (S k) k^T) + b v k^T */
    for (int32_t i = 0; i < Dv; ++i)
      for (int32_t j = 0; j < Dk; ++j) {
        double* s = &S[(int64_t)i * Dk + j];
        *s = decay * (*s - b * Sk[i] * kt[j]) + b * vt[i] * kt[j];
      }
    /* o_t = scale * S q_t */
    double* ot = o + (t * H + h) * (int64_t)Dv;
    for (int32_t i = 0; i < Dv; ++i) {
      double acc = 0.0;
      for (int32_t j = 0; j < Dk; ++j) acc += S[(int64_t)i * Dk + j] * qt[j];
      ot[i] = scale * acc;
    }
  }

  if (ht_nh)
    for (int32_t j = 0; j < Dk; ++j)
      for (int32_t i = 0; i < Dv; ++i) ht_nh[(int64_t)j * Dv + i] = S[(int64_t)i * Dk + j];
}

/* Returns 0 on success, a negative value on a bad argument. */
int gdn_oracle_fwd(int32_t N, const int64_t* start, const int64_t* len, int32_t H,
                   int32_t Hg, int32_t Dk, int32_t Dv, const double* q, const double* k,
                   const double* v, const double* g, const double* beta,
                   const double* h0, double scale, double* o, double* ht,
                   const int64_t* pairs, int64_t n_pairs, int32_t nthreads) {
  if (N < 0 || H <= 0 || Hg <= 0 || Dk <= 0 || Dv <= 0 || H % Hg != 0) return -1;
  if (!start || !len || !q || !k || !v || !g || !beta || !o) return -2;
  const int64_t total = pairs ? n_pairs : (int64_t)N * H;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)Dk * (size_t)Dv);
    double* Sk = (double*)malloc(sizeof(double) * (size_t)Dv);
    if (!S || !Sk) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      bad = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
      for (int64_t p = 0; p < total; ++p) {
        const int64_t pair = pairs ? pairs[p] : p;
        if (pair < 0 || pair >= (int64_t)N * H) continue;
        const int32_t n = (int32_t)(pair / H), h = (int32_t)(pair % H);
        const int64_t off = ((int64_t)n * H + h) * (int64_t)Dk * Dv;
        run_pair(start[n], len[n], h, H, Hg, Dk, Dv, q, k, v, g, beta,
                 h0 ? h0 + off : NULL, scale, o, ht ? ht + off : NULL, S, Sk);
      }
    }
    free(S);
    free(Sk);
  }
  return bad ? -3 : 0;
}

/* Number of threads an OpenMP region would use (for reporting the CPU baseline). */
int gdn_oracle_max_threads(int32_t nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}
