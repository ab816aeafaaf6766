/*
 * ttt_oracle.c -- plain fp64 CPU oracle of the In-Place TTT fast-weight MLP layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only the
 * test suite, the package smoke check and the benchmark's CPU-baseline leg load
 * it.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes, and where that is written down (page "In-Place TTT：给LLM装上
 * '临时记忆插槽'，让它边读边学", zhichai.net):
 *   - section 3.1: the gated MLP  O = phi(H W_gate^T) (.) (H W_up^T) W_down^T ; the
 *     gate phi is taken to be SiLU, phi(x) = x / (1 + exp(-x)).
 *   - section 3.2: the chunk-wise schedule.  A chunk's output is made with the
 *     current fast weight; after the chunk the weight takes one update; the next
 *     chunk uses the updated weight.  Also the three-step parallel form: every
 *     chunk's increment dW_i = V_i^T Z_i, one prefix sum, then every chunk applies
 *     its effective weight.
 *   - section 3.3: the LM-aligned target  V^ = Conv1D(X0) W_target  and the update
 *     W^(i) = W^(i-1) + eta V^_i^T Z_i  (one gradient step on L = -<V^, Z W^T>_F).
 * The same chunk flow is described in prose on the xiaoxiang.io summary of the
 * paper ("原位测试时训练", section 3 "高效的块状更新机制").
 *
 * Readings taken where the page is loose (each is listed in the design notes):
 *   - Conv1D is depthwise with K taps: U[t][c] = sum_k taps[c][k] * X0[t+1-k][c],
 *     k = 0..K-1, so tap 0 looks one token ahead (the next-token alignment of the
 *     page's Theorem 1 discussion, section 4).  X0 is zero outside [0, T) of each
 *     sequence; the conv runs over the whole sequence, not restarted per chunk.
 *     No bias, no activation.
 *   - W_target is d x d, stored [c_in][j_out], applied on the right: V^ = U W_target.
 *   - eta is a plain scalar: no 1/C normalisation, no decay, no clipping.
 *   - Chunk i (0-based) uses W^(i-1); chunk 0 uses W_down0; the last chunk's
 *     update is part of the returned final weight.  A tail chunk shorter than C
 *     follows the same rules.
 *   - Batched sequences are independent: own state, own padding, shared weights.
 *
 * Number format: every input arrives as float32 holding the exact value of the
 * bf16 / fp32 input; every operation here is in double.  Nothing is rounded to a
 * narrower type.  Loops are written in the order the definitions state them;
 * OpenMP only splits independent outputs across threads (each output's sum runs
 * in one thread in index order), so results do not depend on the thread count.
 *
 * Parity status of each entry point is stated in the test suite's oracle pins;
 * every function below has at least one independent pin.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

static double silu(double x) { return x / (1.0 + exp(-x)); }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Gated activations of section 3.1 for `rows` token rows:
 *   Z[t][n] = silu( sum_c H[t][c] Wg[n][c] ) * ( sum_c H[t][c] Wu[n][c] ).
 * H [rows][d], Wg/Wu [f][d], Z [rows][f]. */
void oracle_gated_activations(int64_t rows, int64_t d, int64_t f, const float* H,
                              const float* Wg, const float* Wu, double* Z) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < rows; ++t) {
    const float* h = H + t * d;
    for (int64_t n = 0; n < f; ++n) {
      const float* g = Wg + n * d;
      const float* u = Wu + n * d;
      double a = 0.0, b = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        a += (double)h[c] * (double)g[c];
        b += (double)h[c] * (double)u[c];
      }
      Z[t * f + n] = silu(a) * b;
    }
  }
}

/* The depthwise causal conv of section 3.3 for one sequence of T tokens, at token
 * rows [r0, r1):  U[t][c] = sum_{k=0}^{K-1} taps[c][k] * X0[t+1-k][c],
 * with X0[s] = 0 for s < 0 or s >= T.  X0 [T][d], taps [d][K], U [r1-r0][d]. */
static void conv_rows(int64_t T, int64_t d, int32_t K, int64_t r0, int64_t r1,
                      const float* X0, const float* taps, double* U) {
#pragma omp parallel for schedule(static)
  for (int64_t t = r0; t < r1; ++t) {
    for (int64_t c = 0; c < d; ++c) {
      double s = 0.0;
      for (int32_t k = 0; k < K; ++k) {
        int64_t src = t + 1 - k;
        if (src < 0 || src >= T) continue; /* zero padding at both ends */
        s += (double)taps[c * K + k] * (double)X0[src * d + c];
      }
      U[(t - r0) * d + c] = s;
    }
  }
}

/* V^[t][j] = sum_c U[t][c] Wt[c][j] for `rows` rows.  U [rows][d], Wt [d][d]. */
static void project_rows(int64_t rows, int64_t d, const double* U, const float* Wt,
                         double* V) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < rows; ++t) {
    for (int64_t j = 0; j < d; ++j) {
      double s = 0.0;
      for (int64_t c = 0; c < d; ++c) s += U[t * d + c] * (double)Wt[c * d + j];
      V[t * d + j] = s;
    }
  }
}

/* LM-aligned target V^ = Conv1D(X0) W_target (section 3.3) for B independent
 * sequences of T tokens.  X0 [B][T][d], taps [d][K], Wt [d][d], V [B][T][d]. */
int oracle_lm_target(int64_t B, int64_t T, int64_t d, int32_t K, const float* X0,
                     const float* taps, const float* Wt, double* V) {
  if (B < 1 || T < 1 || d < 1 || K < 1) return ORACLE_EINVAL;
  double* U = (double*)malloc((size_t)(T * d) * sizeof(double));
  if (!U) return ORACLE_ENOMEM;
  for (int64_t b = 0; b < B; ++b) {
    conv_rows(T, d, K, 0, T, X0 + b * T * d, taps, U);
    project_rows(T, d, U, Wt, V + b * T * d);
  }
  free(U);
  return ORACLE_OK;
}

/* Sequential scan (section 3.2 schedule, section 3.3 rule), one sequence, streamed
 * chunk by chunk (memory O(C*(d+f) + d*f)).  W is [d][f] and holds W^(0) on
 * entry, W^(N) on exit.  Per chunk i over rows r in [iC, min(iC+C, T)):
 *   first   O[r][m] = sum_n Z[r][n] W[m][n]            (output with W^(i-1))
 *   then    W[m][n] += eta * sum_r V^[r][m] Z[r][n]    (W^(i) = W^(i-1) + eta V^_i^T Z_i)
 */
/* Progress report (for runs of minutes): a line on stderr every
 * g_progress_every chunks of the sequential form; 0 = silent.  No effect on
 * the arithmetic. */
static int64_t g_progress_every = 0;
void oracle_set_progress(int64_t every) { g_progress_every = every; }

static int sequential_one(int64_t T, int64_t d, int64_t f, int64_t C, int32_t K,
                          double eta, const float* H, const float* X0, const float* Wg,
                          const float* Wu, const float* taps, const float* Wt,
                          double* O, double* W) {
  double* Zc = (double*)malloc((size_t)(C * f) * sizeof(double));
  double* Uc = (double*)malloc((size_t)(C * d) * sizeof(double));
  double* Vc = (double*)malloc((size_t)(C * d) * sizeof(double));
  if (!Zc || !Uc || !Vc) {
    free(Zc); free(Uc); free(Vc);
    return ORACLE_ENOMEM;
  }
  for (int64_t r0 = 0; r0 < T; r0 += C) {
    const int64_t r1 = (r0 + C < T) ? r0 + C : T;
    const int64_t rows = r1 - r0;
    oracle_gated_activations(rows, d, f, H + r0 * d, Wg, Wu, Zc);
    conv_rows(T, d, K, r0, r1, X0, taps, Uc);
    project_rows(rows, d, Uc, Wt, Vc);
    /* output of this chunk with the weight as it stands */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t m = 0; m < d; ++m) {
        double s = 0.0;
        for (int64_t n = 0; n < f; ++n) s += Zc[r * f + n] * W[m * f + n];
        O[(r0 + r) * d + m] = s;
      }
    }
    /* then one update with this chunk's target and activations */
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < d; ++m) {
      for (int64_t n = 0; n < f; ++n) {
        double s = 0.0;
        for (int64_t r = 0; r < rows; ++r) s += Vc[r * d + m] * Zc[r * f + n];
        W[m * f + n] += eta * s;
      }
    }
    const int64_t done = r0 / C + 1;
    if (g_progress_every > 0 && done % g_progress_every == 0) {
      fprintf(stderr, "[oracle] chunk %lld of %lld\n", (long long)done,
              (long long)((T + C - 1) / C));
      fflush(stderr);
    }
  }
  free(Zc); free(Uc); free(Vc);
  return ORACLE_OK;
}

static int check_shape(int64_t B, int64_t T, int64_t d, int64_t f, int64_t C, int32_t K) {
  return (B >= 1 && T >= 1 && d >= 1 && f >= 1 && C >= 1 && K >= 1) ? ORACLE_OK
                                                                     : ORACLE_EINVAL;
}

/* Sequential form for B independent sequences.
 * H, X0 [B][T][d]; Wg, Wu [f][d]; taps [d][K]; Wt [d][d];
 * W_init [B][d][f] (each sequence's starting fast weight);
 * O [B][T][d]; W_out [B][d][f] receives each sequence's final weight. */
int oracle_forward_sequential(int64_t B, int64_t T, int64_t d, int64_t f, int64_t C,
                              int32_t K, double eta, const float* H, const float* X0,
                              const float* Wg, const float* Wu, const float* W_init,
                              const float* taps, const float* Wt, double* O,
                              double* W_out) {
  int rc = check_shape(B, T, d, f, C, K);
  if (rc) return rc;
  for (int64_t b = 0; b < B; ++b) {
    double* W = W_out + b * d * f;
    for (int64_t i = 0; i < d * f; ++i) W[i] = (double)W_init[b * d * f + i];
    rc = sequential_one(T, d, f, C, K, eta, H + b * T * d, X0 + b * T * d, Wg, Wu, taps,
                        Wt, O + b * T * d, W);
    if (rc) return rc;
  }
  return ORACLE_OK;
}

/* Chunk-parallel form, the three steps of section 3.2, one sequence:
 *   step 1: dW_i = V^_i^T Z_i for every chunk i (all materialised);
 *   step 2: exclusive prefix P_i = sum_{j<i} dW_j;
 *   step 3: every chunk applies W_eff^(i) = W^(0) + eta P_i:  O_i = Z_i W_eff^(i)^T.
 * The final weight is W^(0) + eta * (P_{N-1} + dW_{N-1}).  Memory O(N*d*f). */
static int parallel_one(int64_t T, int64_t d, int64_t f, int64_t C, int32_t K, double eta,
                        const float* H, const float* X0, const float* Wg, const float* Wu,
                        const float* W0, const float* taps, const float* Wt, double* O,
                        double* W_final) {
  const int64_t N = (T + C - 1) / C;
  double* Z = (double*)malloc((size_t)(T * f) * sizeof(double));
  double* V = (double*)malloc((size_t)(T * d) * sizeof(double));
  double* dW = (double*)malloc((size_t)(N * d * f) * sizeof(double));
  double* P = (double*)malloc((size_t)(N * d * f) * sizeof(double));
  double* Weff = (double*)malloc((size_t)(d * f) * sizeof(double));
  if (!Z || !V || !dW || !P || !Weff) {
    free(Z); free(V); free(dW); free(P); free(Weff);
    return ORACLE_ENOMEM;
  }
  oracle_gated_activations(T, d, f, H, Wg, Wu, Z);
  int rc = oracle_lm_target(1, T, d, K, X0, taps, Wt, V);
  if (rc) {
    free(Z); free(V); free(dW); free(P); free(Weff);
    return rc;
  }
  /* step 1: independent per-chunk increments */
  for (int64_t i = 0; i < N; ++i) {
    const int64_t r0 = i * C, r1 = (r0 + C < T) ? r0 + C : T;
    double* D = dW + i * d * f;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < d; ++m)
      for (int64_t n = 0; n < f; ++n) {
        double s = 0.0;
        for (int64_t r = r0; r < r1; ++r) s += V[r * d + m] * Z[r * f + n];
        D[m * f + n] = s;
      }
  }
  /* step 2: one exclusive prefix sum over the chunk axis */
  for (int64_t e = 0; e < d * f; ++e) P[e] = 0.0;
  for (int64_t i = 1; i < N; ++i)
    for (int64_t e = 0; e < d * f; ++e)
      P[i * d * f + e] = P[(i - 1) * d * f + e] + dW[(i - 1) * d * f + e];
  /* step 3: each chunk applies its effective weight */
  for (int64_t i = 0; i < N; ++i) {
    const int64_t r0 = i * C, r1 = (r0 + C < T) ? r0 + C : T;
    for (int64_t e = 0; e < d * f; ++e) Weff[e] = (double)W0[e] + eta * P[i * d * f + e];
#pragma omp parallel for schedule(static)
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t m = 0; m < d; ++m) {
        double s = 0.0;
        for (int64_t n = 0; n < f; ++n) s += Z[r * f + n] * Weff[m * f + n];
        O[r * d + m] = s;
      }
  }
  for (int64_t e = 0; e < d * f; ++e)
    W_final[e] = (double)W0[e] + eta * (P[(N - 1) * d * f + e] + dW[(N - 1) * d * f + e]);
  free(Z); free(V); free(dW); free(P); free(Weff);
  return ORACLE_OK;
}

int oracle_forward_chunk_parallel(int64_t B, int64_t T, int64_t d, int64_t f, int64_t C,
                                  int32_t K, double eta, const float* H, const float* X0,
                                  const float* Wg, const float* Wu, const float* W_init,
                                  const float* taps, const float* Wt, double* O,
                                  double* W_out) {
  int rc = check_shape(B, T, d, f, C, K);
  if (rc) return rc;
  for (int64_t b = 0; b < B; ++b) {
    rc = parallel_one(T, d, f, C, K, eta, H + b * T * d, X0 + b * T * d, Wg, Wu,
                      W_init + b * d * f, taps, Wt, O + b * T * d, W_out + b * d * f);
    if (rc) return rc;
  }
  return ORACLE_OK;
}

/* Dual form, for small shapes.  Unrolling the update rule gives, for a token t in
 * chunk i (chunk start c(t) = C * floor(t / C)),
 *   W^(i-1) = W^(0) + eta * sum_{s < c(t)} V^[s]^T Z[s]
 *   O[t]    = Z[t] W^(0)^T + eta * sum_{s < c(t)} (Z[t] . Z[s]) V^[s],
 * and the final weight is the closed form W^(0) + eta * sum_{all s} V^[s]^T Z[s].
 * This is an algebraic consequence of the section 3.3 rule, not a form the page
 * prints; it shares no loop structure with the two scans above. */
static int dual_one(int64_t T, int64_t d, int64_t f, int64_t C, int32_t K, double eta,
                    const float* H, const float* X0, const float* Wg, const float* Wu,
                    const float* W0, const float* taps, const float* Wt, double* O,
                    double* W_final) {
  double* Z = (double*)malloc((size_t)(T * f) * sizeof(double));
  double* V = (double*)malloc((size_t)(T * d) * sizeof(double));
  if (!Z || !V) {
    free(Z); free(V);
    return ORACLE_ENOMEM;
  }
  oracle_gated_activations(T, d, f, H, Wg, Wu, Z);
  int rc = oracle_lm_target(1, T, d, K, X0, taps, Wt, V);
  if (rc) {
    free(Z); free(V);
    return rc;
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const int64_t ct = C * (t / C);
    for (int64_t m = 0; m < d; ++m) {
      double s = 0.0;
      for (int64_t n = 0; n < f; ++n) s += Z[t * f + n] * (double)W0[m * f + n];
      O[t * d + m] = s;
    }
    for (int64_t s = 0; s < ct; ++s) {
      double kz = 0.0;
      for (int64_t n = 0; n < f; ++n) kz += Z[t * f + n] * Z[s * f + n];
      for (int64_t m = 0; m < d; ++m) O[t * d + m] += eta * kz * V[s * d + m];
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < d; ++m)
    for (int64_t n = 0; n < f; ++n) {
      double s = 0.0;
      for (int64_t r = 0; r < T; ++r) s += V[r * d + m] * Z[r * f + n];
      W_final[m * f + n] = (double)W0[m * f + n] + eta * s;
    }
  free(Z); free(V);
  return ORACLE_OK;
}

int oracle_forward_dual(int64_t B, int64_t T, int64_t d, int64_t f, int64_t C, int32_t K,
                        double eta, const float* H, const float* X0, const float* Wg,
                        const float* Wu, const float* W_init, const float* taps,
                        const float* Wt, double* O, double* W_out) {
  int rc = check_shape(B, T, d, f, C, K);
  if (rc) return rc;
  for (int64_t b = 0; b < B; ++b) {
    rc = dual_one(T, d, f, C, K, eta, H + b * T * d, X0 + b * T * d, Wg, Wu,
                  W_init + b * d * f, taps, Wt, O + b * T * d, W_out + b * d * f);
    if (rc) return rc;
  }
  return ORACLE_OK;
}

/* Selected entries of the final weight of ONE sequence by the closed form
 *   W^(N)[m][n] = W^(0)[m][n] + eta * sum_{t<T} V^[t][m] * Z[t][n],
 * on the grid ms[0..nm) x ns[0..nn) -> out[nm][nn].  Each needed column of Z and
 * of V^ is computed on its own over all T tokens (memory O(T)), so this serves
 * shapes whose full Z and V^ would not fit.  H, X0 [T][d]; W0 [d][f]. */
int oracle_final_weight_grid(int64_t T, int64_t d, int64_t f, int32_t K, double eta,
                             const float* H, const float* X0, const float* Wg,
                             const float* Wu, const float* W0, const float* taps,
                             const float* Wt, int64_t nm, const int64_t* ms, int64_t nn,
                             const int64_t* ns, double* out) {
  if (T < 1 || d < 1 || f < 1 || K < 1 || nm < 0 || nn < 0) return ORACLE_EINVAL;
  for (int64_t a = 0; a < nm; ++a)
    if (ms[a] < 0 || ms[a] >= d) return ORACLE_EINVAL;
  for (int64_t a = 0; a < nn; ++a)
    if (ns[a] < 0 || ns[a] >= f) return ORACLE_EINVAL;
  double* zc = (double*)malloc((size_t)(nn * T) * sizeof(double));
  double* vc = (double*)malloc((size_t)(nm * T) * sizeof(double));
  if (!zc || !vc) {
    free(zc); free(vc);
    return ORACLE_ENOMEM;
  }
  /* Z[:, n] for each requested n */
  for (int64_t a = 0; a < nn; ++a) {
    const int64_t n = ns[a];
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      double g = 0.0, u = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        g += (double)H[t * d + c] * (double)Wg[n * d + c];
        u += (double)H[t * d + c] * (double)Wu[n * d + c];
      }
      zc[a * T + t] = silu(g) * u;
    }
  }
  /* V^[:, m] for each requested m, with the conv evaluated on the fly */
  for (int64_t a = 0; a < nm; ++a) {
    const int64_t m = ms[a];
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      double v = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        double uc = 0.0;
        for (int32_t k = 0; k < K; ++k) {
          int64_t src = t + 1 - k;
          if (src < 0 || src >= T) continue;
          uc += (double)taps[c * K + k] * (double)X0[src * d + c];
        }
        v += uc * (double)Wt[c * d + m];
      }
      vc[a * T + t] = v;
    }
  }
  for (int64_t a = 0; a < nm; ++a)
    for (int64_t b = 0; b < nn; ++b) {
      double s = 0.0;
      for (int64_t t = 0; t < T; ++t) s += vc[a * T + t] * zc[b * T + t];
      out[a * nn + b] = (double)W0[ms[a] * f + ns[b]] + eta * s;
    }
  free(zc); free(vc);
  return ORACLE_OK;
}
