/*
 * CPU oracle for the multi-round dropless mixture-of-experts layer: forward,
 * and the backward of its plain definition.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this file's library. The HIP
 * library never links, includes or calls it, and it shares no code with the
 * HIP library: no headers, kernels, helpers or tables.
 *
 * Everything is computed in fp64 with plain loops, in the order of the
 * definitions below, so that a reader can check it against the sources:
 *
 *   [P1] "Frontier Pre-training at Microsoft AI (MAI-Base-2)", section
 *        "Key claims", item on multi-round dropless MoE (quoting the post's
 *        section "Scaling MoE", Fig. 6).
 *   [P3] "MAI-Base-2: Microsoft details its new training infrastructure",
 *        section "Optimizations to prevent memory loss".
 *   [P4] "Microsoft AI's MAI-Base-2 trained on 16K GPUs with Muon", section
 *        "Expert groups keep memory fixed when tokens pile up".
 *   [P2] "MAI-Base-2: Microsoft's 2.8T Model is a BREAKTHROUGH", video
 *        transcript at 03:11.
 *
 * The pages give the method only in outline: routing assigns every token to
 * a small number of experts; the experts of a group then work in rounds of
 * dispatch, compute and collect, each round holding at most a fixed number
 * of tokens per expert; assignments that do not fit are deferred to a later
 * round, so none is lost. Where they are silent this file takes these readings:
 *   - routing is top-k over the raw logits with ties to the lower expert
 *     index, and the k weights are the softmax over all E logits
 *     renormalised over the k chosen experts;
 *   - an expert's assignments keep ascending token order (stable), and the
 *     first C of them go to round 0, the next C to round 1, and so on;
 *   - round-buffer row of the c-th slot of expert e is e*C + c, where a
 *     capacity above T acts as T (an expert never holds more than T tokens);
 *   - the expert FFN is SwiGLU with no biases: h = silu(x.Wg^T) * (x.Wu^T),
 *     o = h.Wd^T; the layer output is y_t = sum_j w_tj * o_tj, j ascending;
 *   - with capacity shared in groups of G experts (oracle_plan_groups), an
 *     expert first fills its own C slots, then the group's unused slots go
 *     to its overloaded experts in ascending expert order.
 *
 * Parity pins for every function live in the test suite (brute-force top-k,
 * library sort/histogram, closed forms, a library SwiGLU for E = k = 1,
 * bit-identity of the round executors with the per-token loop for every C
 * and group size, a Python simulation of the group fill rule, and
 * hand-worked fixtures; for the backward, central finite differences of
 * the forward for every gradient entry of a small layer, a library
 * autograd of the SwiGLU FFN for E = k = 1, and router-gradient
 * identities).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_ARG -1
#define OR_ERR_NONFINITE -2
#define OR_ERR_PLAN -3
#define OR_ERR_NOMEM -4

static int64_t min_i64(int64_t a, int64_t b) { return a < b ? a : b; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Router [P4 "Expert groups keep memory fixed..."]: every token is routed to
 * a small number of experts. Top-k by raw fp32 logit, order (logit descending, expert index
 * ascending); -0 and +0 compare equal. Then the softmax over all E logits,
 * renormalised over the k chosen experts. idx is [T][k] int32, w is [T][k]
 * fp64. Returns OR_ERR_NONFINITE if any logit is NaN or infinite. */
int oracle_route(int64_t T, int32_t E, int32_t k, const float *logits,
                 int32_t *idx, double *w) {
  if (T < 1 || E < 1 || k < 1 || k > E || !logits || !idx || !w)
    return OR_ERR_ARG;
  for (int64_t i = 0; i < T * (int64_t)E; ++i)
    if (!isfinite(logits[i])) return OR_ERR_NONFINITE;
  int err = OR_OK;
#pragma omp parallel
  {
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    if (!taken || !p) {
#pragma omp atomic write
      err = OR_ERR_NOMEM;
    } else {
#pragma omp for schedule(static)
      for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        /* selection: the j-th pick is the best expert not yet taken */
        for (int32_t j = 0; j < k; ++j) {
          int32_t best = -1;
          for (int32_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            /* strictly greater wins; equal keeps the lower index found first */
            if (best < 0 || l[e] > l[best]) best = e;
          }
          taken[best] = 1;
          idx[t * k + j] = best;
        }
        /* softmax over all E in fp64 (max subtracted), then renormalise */
        double mx = (double)l[0];
        for (int32_t e = 1; e < E; ++e)
          if ((double)l[e] > mx) mx = (double)l[e];
        double z = 0.0;
        for (int32_t e = 0; e < E; ++e) {
          p[e] = exp((double)l[e] - mx);
          z += p[e];
        }
        for (int32_t e = 0; e < E; ++e) p[e] /= z;
        double s = 0.0;
        for (int32_t j = 0; j < k; ++j) s += p[idx[t * k + j]];
        for (int32_t j = 0; j < k; ++j) w[t * k + j] = p[idx[t * k + j]] / s;
      }
    }
    free(taken);
    free(p);
  }
  return err;
}

/* Plan [P1 "Key claims", P4, P3 "Optimizations to prevent memory loss"]:
 * per-expert token counts, the stable permutation of assignment ids
 * a = t*k + j sorted by expert (ascending a inside an expert), its inverse,
 * and the split of each expert's list into rounds of at most C:
 *   i = pos[a] - offsets[e];  round_of[a] = i / C;  row_of[a] = e*C + i % C
 *   R = max_e ceil(counts[e] / C).
 * A capacity above T acts as T. */
int oracle_plan(int64_t T, int32_t E, int32_t k, int64_t C, const int32_t *idx,
                int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *pos,
                int32_t *round_of, int32_t *row_of, int32_t *R) {
  if (T < 1 || E < 1 || k < 1 || k > E || C < 1 || !idx || !counts ||
      !offsets || !perm || !pos || !round_of || !row_of || !R)
    return OR_ERR_ARG;
  const int64_t TK = T * k;
  const int64_t Ce = min_i64(C, T);
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < TK; ++a) {
    if (idx[a] < 0 || idx[a] >= E) return OR_ERR_ARG;
    counts[idx[a]] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  /* counting sort, scanning a upward keeps each expert's list stable */
  int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  if (!cursor) return OR_ERR_NOMEM;
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t a = 0; a < TK; ++a) perm[cursor[idx[a]]++] = (int32_t)a;
  free(cursor);
  for (int64_t p = 0; p < TK; ++p) pos[perm[p]] = (int32_t)p;
  for (int64_t a = 0; a < TK; ++a) {
    const int32_t e = idx[a];
    const int64_t i = (int64_t)pos[a] - offsets[e];
    round_of[a] = (int32_t)(i / Ce);
    row_of[a] = (int32_t)((int64_t)e * Ce + i % Ce);
  }
  int32_t rmax = 0;
  for (int32_t e = 0; e < E; ++e) {
    const int32_t r = (int32_t)((counts[e] + Ce - 1) / Ce);
    if (r > rmax) rmax = r;
  }
  *R = rmax;
  return OR_OK;
}

/* Expert FFN of one row [P1 "Key claims": dispatch -> compute -> collect;
 * SwiGLU with no biases]. xr is the token row in fp64; Wg_e, Wu_e are
 * [f][d], Wd_e is [d][f]. h (length f) receives silu(g)*u, o (length d)
 * receives h.Wd^T. Sums run over ascending index, no intermediate rounding. */
/*
 * Plan with capacity shared inside expert groups ("Frontier Pre-training at
 * Microsoft AI (MAI-Base-2)", section "Key claims", and "Microsoft AI's
 * MAI-Base-2 trained on 16K GPUs with Muon", section "Expert groups keep
 * memory fixed when tokens pile up": an overloaded expert first uses the
 * unused capacity of the other experts of its group, and only what still
 * does not fit waits for another round).
 *
 * Reading taken here (the pages give no procedure): experts e are grouped
 * by e / G (G consecutive experts, G divides E). In every round a group
 * owns G * C' slots. Each expert first takes min(remaining, C') of its
 * remaining assignments (its own capacity); the slots its group leaves
 * unused then go to the group's overloaded experts in ascending expert
 * order, each taking as many of its remaining assignments as the spare
 * slots allow. An expert's assignments keep their stable order and each
 * round takes the next m(r, e) of them. Inside a round the group's slots
 * are filled expert by expert: row_of = g * G * C' + (rows of the group's
 * lower experts in that round) + c. G = 1 is the strict per-expert
 * capacity of oracle_plan.
 *
 * alloc receives m(r, e) for r < *R (alloc_rows * E int32 provided).
 */
int oracle_plan_groups(int64_t T, int32_t E, int32_t k, int64_t C, int32_t G,
                       const int32_t *idx, int32_t *counts, int32_t *offsets,
                       int32_t *perm, int32_t *pos, int32_t *round_of,
                       int32_t *row_of, int32_t *R, int32_t *alloc,
                       int64_t alloc_rows) {
  if (T < 1 || E < 1 || k < 1 || k > E || C < 1 || G < 1 || E % G != 0 ||
      !idx || !counts || !offsets || !perm || !pos || !round_of || !row_of ||
      !R || !alloc || alloc_rows < 1)
    return OR_ERR_ARG;
  const int64_t TK = T * k;
  const int64_t Ce = min_i64(C, T);
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < TK; ++a) {
    if (idx[a] < 0 || idx[a] >= E) return OR_ERR_ARG;
    counts[idx[a]] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int64_t *rem = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
  if (!cursor || !rem) {
    free(cursor);
    free(rem);
    return OR_ERR_NOMEM;
  }
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t a = 0; a < TK; ++a) perm[cursor[idx[a]]++] = (int32_t)a;
  for (int64_t p = 0; p < TK; ++p) pos[perm[p]] = (int32_t)p;

  /* rounds: allocation table m(r, e) */
  for (int32_t e = 0; e < E; ++e) rem[e] = counts[e];
  int64_t r = 0;
  int err = OR_OK;
  for (;;) {
    int64_t left = 0;
    for (int32_t e = 0; e < E; ++e) left += rem[e];
    if (left == 0) break;
    if (r >= alloc_rows) {
      err = OR_ERR_ARG;
      break;
    }
    int32_t *m = alloc + r * E;
    for (int32_t g0 = 0; g0 < E; g0 += G) {
      int64_t spare = (int64_t)G * Ce;
      for (int32_t e = g0; e < g0 + G; ++e) {
        m[e] = (int32_t)min_i64(rem[e], Ce);
        spare -= m[e];
      }
      for (int32_t e = g0; e < g0 + G; ++e) {
        const int64_t more = min_i64(rem[e] - m[e], spare);
        m[e] += (int32_t)more;
        spare -= more;
      }
      for (int32_t e = g0; e < g0 + G; ++e) rem[e] -= m[e];
    }
    ++r;
  }
  *R = (int32_t)r;
  /* each assignment's round and row */
  for (int64_t a = 0; a < TK && err == OR_OK; ++a) {
    const int32_t e = idx[a];
    const int32_t g0 = e - e % G;
    int64_t i = (int64_t)pos[a] - offsets[e]; /* index in expert e's list */
    int64_t rr = 0;
    while (i >= alloc[rr * E + e]) {
      i -= alloc[rr * E + e];
      ++rr;
    }
    int64_t before = 0; /* rows of the group's lower experts in round rr */
    for (int32_t e2 = g0; e2 < e; ++e2) before += alloc[rr * E + e2];
    round_of[a] = (int32_t)rr;
    row_of[a] = (int32_t)((int64_t)g0 * Ce + before + i);
  }
  free(cursor);
  free(rem);
  return err;
}

static void expert_ffn_row(int32_t d, int32_t f, const double *xr,
                           const float *Wg_e, const float *Wu_e,
                           const float *Wd_e, double *h, double *o) {
  for (int32_t q = 0; q < f; ++q) {
    const float *wg = Wg_e + (int64_t)q * d;
    const float *wu = Wu_e + (int64_t)q * d;
    double g = 0.0, u = 0.0;
    for (int32_t i = 0; i < d; ++i) {
      g += xr[i] * (double)wg[i];
      u += xr[i] * (double)wu[i];
    }
    h[q] = g / (1.0 + exp(-g)) * u;
  }
  for (int32_t m = 0; m < d; ++m) {
    const float *wd = Wd_e + (int64_t)m * f;
    double acc = 0.0;
    for (int32_t q = 0; q < f; ++q) acc += h[q] * (double)wd[q];
    o[m] = acc;
  }
}

/* Per-assignment expert outputs for a list of assignment ids: h[n][f] (may
 * be NULL) and o[n][d]. Used to check the per-round intermediate buffers. */
int oracle_assignment_outputs(int64_t T, int32_t E, int32_t k, int32_t d,
                              int32_t f, int64_t n, const int64_t *a_list,
                              const int32_t *idx, const float *x,
                              const float *Wg, const float *Wu,
                              const float *Wd, double *h_out, double *o_out) {
  if (T < 1 || E < 1 || k < 1 || d < 1 || f < 1 || n < 0 || !a_list ||
      !idx || !x || !Wg || !Wu || !Wd || !o_out)
    return OR_ERR_ARG;
  for (int64_t s = 0; s < n; ++s)
    if (a_list[s] < 0 || a_list[s] >= T * k) return OR_ERR_ARG;
  int err = OR_OK;
#pragma omp parallel
  {
    double *xr = (double *)malloc(sizeof(double) * (size_t)d);
    double *h = (double *)malloc(sizeof(double) * (size_t)f);
    if (!xr || !h) {
#pragma omp atomic write
      err = OR_ERR_NOMEM;
    } else {
#pragma omp for schedule(static)
      for (int64_t s = 0; s < n; ++s) {
        const int64_t a = a_list[s];
        const int64_t t = a / k;
        const int32_t e = idx[a];
        for (int32_t i = 0; i < d; ++i) xr[i] = (double)x[t * d + i];
        const int64_t wo = (int64_t)e * f * d;
        expert_ffn_row(d, f, xr, Wg + wo, Wu + wo, Wd + wo, h,
                       o_out + s * d);
        if (h_out) memcpy(h_out + s * f, h, sizeof(double) * (size_t)f);
      }
    }
    free(xr);
    free(h);
  }
  return err;
}

/* The layer as its plain definition, for a list of tokens: for each token,
 * loop over its k experts in j order, run the expert FFN and accumulate
 * y_t = sum_j w_tj * o_tj [P1 "Key claims": collect; weighted sum of the
 * top-k expert outputs]. y is [n][d]. */
int oracle_forward_tokens(int64_t T, int32_t E, int32_t k, int32_t d,
                          int32_t f, int64_t n, const int64_t *tokens,
                          const int32_t *idx, const double *w, const float *x,
                          const float *Wg, const float *Wu, const float *Wd,
                          double *y) {
  if (T < 1 || E < 1 || k < 1 || d < 1 || f < 1 || n < 0 || !tokens ||
      !idx || !w || !x || !Wg || !Wu || !Wd || !y)
    return OR_ERR_ARG;
  for (int64_t s = 0; s < n; ++s)
    if (tokens[s] < 0 || tokens[s] >= T) return OR_ERR_ARG;
  int err = OR_OK;
#pragma omp parallel
  {
    double *xr = (double *)malloc(sizeof(double) * (size_t)d);
    double *h = (double *)malloc(sizeof(double) * (size_t)f);
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    if (!xr || !h || !o) {
#pragma omp atomic write
      err = OR_ERR_NOMEM;
    } else {
#pragma omp for schedule(static)
      for (int64_t s = 0; s < n; ++s) {
        const int64_t t = tokens[s];
        double *yt = y + s * d;
        for (int32_t i = 0; i < d; ++i) xr[i] = (double)x[t * d + i];
        for (int32_t m = 0; m < d; ++m) yt[m] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
          const int32_t e = idx[t * k + j];
          const int64_t wo = (int64_t)e * f * d;
          expert_ffn_row(d, f, xr, Wg + wo, Wu + wo, Wd + wo, h, o);
          for (int32_t m = 0; m < d; ++m) yt[m] += w[t * k + j] * o[m];
        }
      }
    }
    free(xr);
    free(h);
    free(o);
  }
  return err;
}

/* The method itself, executed as the pages describe it [P1 "Key claims",
 * P4, P2 03:11]: for r = 0..R-1, dispatch every round-r assignment into a
 * fixed E x C round buffer (row e*C + c), compute each filled slot's expert
 * FFN, and collect the output into the token-slot buffer Z[a] (T*k rows,
 * initialised to NaN so a dropped slot shows). Finally combine
 * y_t = sum_j w_tj * Z[t*k + j], j ascending. The plan is taken as input and
 * cross-checked: a slot whose round_of/row_of disagrees with its position is
 * an error, as is an assignment that ends unfilled or filled twice.
 * Z is [T*k][d] and y is [T][d]; the round buffer is allocated here with
 * E*min(C,T)*d entries, the same for every routing. */
int oracle_round_executor(int64_t T, int32_t E, int32_t k, int32_t d,
                          int32_t f, int64_t C, const int32_t *idx,
                          const double *w, const int32_t *counts,
                          const int32_t *offsets, const int32_t *perm,
                          const int32_t *round_of, const int32_t *row_of,
                          int32_t R, const float *x, const float *Wg,
                          const float *Wu, const float *Wd, double *Z,
                          double *y) {
  if (T < 1 || E < 1 || k < 1 || d < 1 || f < 1 || C < 1 || R < 0 || !idx ||
      !w || !counts || !offsets || !perm || !round_of || !row_of || !x ||
      !Wg || !Wu || !Wd || !Z || !y)
    return OR_ERR_ARG;
  const int64_t TK = T * k;
  const int64_t Ce = min_i64(C, T);
  const double nan = NAN;
  for (int64_t i = 0; i < TK * d; ++i) Z[i] = nan;
  unsigned char *filled = (unsigned char *)calloc((size_t)TK, 1);
  double *Xr = (double *)malloc(sizeof(double) * (size_t)(E * Ce * d));
  int64_t *slot_a = (int64_t *)malloc(sizeof(int64_t) * (size_t)(E * Ce));
  if (!filled || !Xr || !slot_a) {
    free(filled);
    free(Xr);
    free(slot_a);
    return OR_ERR_NOMEM;
  }
  int err = OR_OK;
  for (int32_t r = 0; r < R && err == OR_OK; ++r) {
    /* dispatch: gather round-r assignments into their fixed slots */
    for (int64_t s = 0; s < E * Ce; ++s) slot_a[s] = -1;
    for (int32_t e = 0; e < E && err == OR_OK; ++e) {
      int64_t m = (int64_t)counts[e] - (int64_t)r * Ce;
      if (m < 0) m = 0;
      if (m > Ce) m = Ce;
      for (int64_t c = 0; c < m; ++c) {
        const int64_t a = perm[offsets[e] + r * Ce + c];
        const int64_t row = (int64_t)e * Ce + c;
        if (idx[a] != e || round_of[a] != r || row_of[a] != row) {
          err = OR_ERR_PLAN;
          break;
        }
        const int64_t t = a / k;
        for (int32_t i = 0; i < d; ++i)
          Xr[row * d + i] = (double)x[t * d + i];
        slot_a[row] = a;
      }
    }
    if (err != OR_OK) break;
    /* compute + collect: each filled slot's expert output goes to Z[a] */
#pragma omp parallel
    {
      double *h = (double *)malloc(sizeof(double) * (size_t)f);
      if (!h) {
#pragma omp atomic write
        err = OR_ERR_NOMEM;
      } else {
#pragma omp for schedule(static)
        for (int64_t row = 0; row < E * Ce; ++row) {
          const int64_t a = slot_a[row];
          if (a < 0) continue;
          const int64_t e = row / Ce;
          const int64_t wo = e * f * d;
          expert_ffn_row(d, f, Xr + row * d, Wg + wo, Wu + wo, Wd + wo, h,
                         Z + a * d);
        }
      }
      free(h);
    }
    for (int64_t row = 0; row < E * Ce && err == OR_OK; ++row) {
      const int64_t a = slot_a[row];
      if (a < 0) continue;
      if (filled[a]) err = OR_ERR_PLAN;
      filled[a] = 1;
    }
  }
  for (int64_t a = 0; a < TK && err == OR_OK; ++a)
    if (!filled[a]) err = OR_ERR_PLAN;
  if (err == OR_OK) {
    /* combine in token order */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      double *yt = y + t * d;
      for (int32_t m = 0; m < d; ++m) yt[m] = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        const double *zr = Z + (t * k + j) * d;
        for (int32_t m = 0; m < d; ++m) yt[m] += w[t * k + j] * zr[m];
      }
    }
  }
  free(filled);
  free(Xr);
  free(slot_a);
  return err;
}

/*
 * Round executor for a plan with shared group capacity (oracle_plan_groups):
 * round by round, the assignments the allocation table gives every expert
 * are gathered into the E * C' slot buffer at their rows, each slot's
 * expert output goes to Z[a] (NaN until written), then the per-token
 * combine. Every row is checked against the table: expert e's m(r, e)
 * slots of round r are the next m(r, e) entries of its list, at rows
 * g * G * C' + (rows of lower experts of its group) + c.
 */
int oracle_round_executor_groups(int64_t T, int32_t E, int32_t k, int32_t d,
                                 int32_t f, int64_t C, int32_t G,
                                 const int32_t *idx, const double *w,
                                 const int32_t *counts, const int32_t *offsets,
                                 const int32_t *perm, const int32_t *round_of,
                                 const int32_t *row_of, int32_t R,
                                 const int32_t *alloc, const float *x,
                                 const float *Wg, const float *Wu,
                                 const float *Wd, double *Z, double *y) {
  if (T < 1 || E < 1 || k < 1 || d < 1 || f < 1 || C < 1 || G < 1 ||
      E % G != 0 || R < 0 || !idx || !w || !counts || !offsets || !perm ||
      !round_of || !row_of || !alloc || !x || !Wg || !Wu || !Wd || !Z || !y)
    return OR_ERR_ARG;
  const int64_t TK = T * k;
  const int64_t Ce = min_i64(C, T);
  const double nan = NAN;
  for (int64_t i = 0; i < TK * d; ++i) Z[i] = nan;
  unsigned char *filled = (unsigned char *)calloc((size_t)TK, 1);
  double *Xr = (double *)malloc(sizeof(double) * (size_t)(E * Ce * d));
  int64_t *slot_a = (int64_t *)malloc(sizeof(int64_t) * (size_t)(E * Ce));
  int64_t *used = (int64_t *)calloc((size_t)E, sizeof(int64_t));
  if (!filled || !Xr || !slot_a || !used) {
    free(filled);
    free(Xr);
    free(slot_a);
    free(used);
    return OR_ERR_NOMEM;
  }
  int err = OR_OK;
  for (int32_t r = 0; r < R && err == OR_OK; ++r) {
    for (int64_t s = 0; s < E * Ce; ++s) slot_a[s] = -1;
    for (int32_t g0 = 0; g0 < E && err == OR_OK; g0 += G) {
      int64_t base = (int64_t)g0 * Ce;
      for (int32_t e = g0; e < g0 + G && err == OR_OK; ++e) {
        const int64_t m = alloc[(int64_t)r * E + e];
        if (m < 0 || base + m > (int64_t)(g0 + G) * Ce ||
            used[e] + m > counts[e]) {
          err = OR_ERR_PLAN;
          break;
        }
        for (int64_t c = 0; c < m; ++c) {
          const int64_t a = perm[offsets[e] + used[e] + c];
          const int64_t row = base + c;
          if (idx[a] != e || round_of[a] != r || row_of[a] != row ||
              slot_a[row] != -1) {
            err = OR_ERR_PLAN;
            break;
          }
          const int64_t t = a / k;
          for (int32_t i = 0; i < d; ++i)
            Xr[row * d + i] = (double)x[t * d + i];
          slot_a[row] = a;
        }
        used[e] += m;
        base += m;
      }
    }
    if (err != OR_OK) break;
#pragma omp parallel
    {
      double *h = (double *)malloc(sizeof(double) * (size_t)f);
      if (!h) {
#pragma omp atomic write
        err = OR_ERR_NOMEM;
      } else {
#pragma omp for schedule(static)
        for (int64_t row = 0; row < E * Ce; ++row) {
          const int64_t a = slot_a[row];
          if (a < 0) continue;
          const int64_t e = idx[a];
          const int64_t wo = e * f * d;
          expert_ffn_row(d, f, Xr + row * d, Wg + wo, Wu + wo, Wd + wo, h,
                         Z + a * d);
        }
      }
      free(h);
    }
    for (int64_t row = 0; row < E * Ce && err == OR_OK; ++row) {
      const int64_t a = slot_a[row];
      if (a < 0) continue;
      if (filled[a]) err = OR_ERR_PLAN;
      filled[a] = 1;
    }
  }
  for (int64_t a = 0; a < TK && err == OR_OK; ++a)
    if (!filled[a]) err = OR_ERR_PLAN;
  if (err == OR_OK) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      double *yt = y + t * d;
      for (int32_t m = 0; m < d; ++m) yt[m] = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        const double *zr = Z + (t * k + j) * d;
        for (int32_t m = 0; m < d; ++m) yt[m] += w[t * k + j] * zr[m];
      }
    }
  }
  free(filled);
  free(Xr);
  free(slot_a);
  free(used);
  return err;
}

/* ------------------------------------------------------------------------
 * Backward of the layer (the gradient of a loss L = sum_t <y_t, dy_t> with
 * respect to x, the expert weights and the router logits), as the plain
 * chain rule of the definition above, in fp64. Where the pages are silent
 * this file reads: the routing selection (top-k) passes no gradient; the k
 * weights are the softmax of the k chosen logits, so only those logits get
 * one; the expert FFN is recomputed from x (nothing but the routing and the
 * unweighted expert outputs is kept from the forward).
 *
 * For one assignment (t, j) with expert e and weight w:
 *   g = x Wg_e^T, u = x Wu_e^T, s = sigmoid(g), a = g s, h = a u,
 *   o = h Wd_e^T;
 *   dw_j = <o, dy_t>;  dO = w dy_t;
 *   dh = dO Wd_e;      dWd_e += dO^T h;
 *   du = dh a;         dg = dh u s (1 + g (1 - s))   (silu'(g));
 *   dWg_e += dg^T x;   dWu_e += du^T x;
 *   dx_t += dg Wg_e + du Wu_e;
 * and for the token: dlogit(e_j) = w_j (dw_j - sum_j' w_j' dw_j'), every
 * other logit 0.
 * ---------------------------------------------------------------------- */

/* The per-assignment recompute and local gradients: fills g, u, a (f) and o
 * (d) for token row xr through expert weights of e. */
static void expert_recompute(int32_t d, int32_t f, const double *xr,
                             const float *Wg_e, const float *Wu_e,
                             const float *Wd_e, double *g, double *u,
                             double *a, double *h, double *o) {
  for (int32_t q = 0; q < f; ++q) {
    const float *wg = Wg_e + (int64_t)q * d;
    const float *wu = Wu_e + (int64_t)q * d;
    double gq = 0.0, uq = 0.0;
    for (int32_t i = 0; i < d; ++i) {
      gq += xr[i] * (double)wg[i];
      uq += xr[i] * (double)wu[i];
    }
    g[q] = gq;
    u[q] = uq;
    a[q] = gq / (1.0 + exp(-gq));
    h[q] = a[q] * uq;
  }
  for (int32_t m = 0; m < d; ++m) {
    const float *wd = Wd_e + (int64_t)m * f;
    double acc = 0.0;
    for (int32_t q = 0; q < f; ++q) acc += h[q] * (double)wd[q];
    o[m] = acc;
  }
}

/* dh = dO Wd_e, then dg and du from the recomputed g, u, a. */
static void expert_dgate(int32_t d, int32_t f, const double *dO,
                         const float *Wd_e, const double *g, const double *u,
                         const double *a, double *dg, double *du) {
  for (int32_t q = 0; q < f; ++q) {
    double dh = 0.0;
    for (int32_t m = 0; m < d; ++m) dh += dO[m] * (double)Wd_e[(int64_t)m * f + q];
    const double s = 1.0 / (1.0 + exp(-g[q]));
    du[q] = dh * a[q];
    dg[q] = dh * u[q] * s * (1.0 + g[q] * (1.0 - s));
  }
}

/* Per-token gradients for a list of tokens: dx [n][d] and dlogits [n][E]. */
int oracle_backward_tokens(int64_t T, int32_t E, int32_t k, int32_t d,
                           int32_t f, int64_t n, const int64_t *tokens,
                           const int32_t *idx, const double *w, const float *x,
                           const float *Wg, const float *Wu, const float *Wd,
                           const float *dy, double *dx, double *dlogits) {
  if (T < 1 || E < 1 || k < 1 || d < 1 || f < 1 || n < 0 || !tokens ||
      !idx || !w || !x || !Wg || !Wu || !Wd || !dy || !dx || !dlogits)
    return OR_ERR_ARG;
  for (int64_t s = 0; s < n; ++s)
    if (tokens[s] < 0 || tokens[s] >= T) return OR_ERR_ARG;
  int err = OR_OK;
#pragma omp parallel
  {
    const size_t F = (size_t)f, D = (size_t)d;
    double *buf = (double *)malloc(sizeof(double) * (6 * F + 3 * D + (size_t)k));
    if (!buf) {
#pragma omp atomic write
      err = OR_ERR_NOMEM;
    } else {
      double *g = buf, *u = g + F, *a = u + F, *h = a + F, *dg = h + F,
             *du = dg + F, *xr = du + F, *o = xr + D, *dO = o + D,
             *dw = dO + D;
#pragma omp for schedule(static)
      for (int64_t s = 0; s < n; ++s) {
        const int64_t t = tokens[s];
        double *dxt = dx + s * d;
        double *dlt = dlogits + s * E;
        for (int32_t i = 0; i < d; ++i) {
          xr[i] = (double)x[t * d + i];
          dxt[i] = 0.0;
        }
        for (int32_t e = 0; e < E; ++e) dlt[e] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
          const int32_t e = idx[t * k + j];
          const int64_t wo = (int64_t)e * f * d;
          const double wj = w[t * k + j];
          expert_recompute(d, f, xr, Wg + wo, Wu + wo, Wd + wo, g, u, a, h, o);
          double acc = 0.0;
          for (int32_t m = 0; m < d; ++m) {
            acc += o[m] * (double)dy[t * d + m];
            dO[m] = wj * (double)dy[t * d + m];
          }
          dw[j] = acc;
          expert_dgate(d, f, dO, Wd + wo, g, u, a, dg, du);
          for (int32_t i = 0; i < d; ++i) {
            double v = 0.0;
            for (int32_t q = 0; q < f; ++q)
              v += dg[q] * (double)Wg[wo + (int64_t)q * d + i] +
                   du[q] * (double)Wu[wo + (int64_t)q * d + i];
            dxt[i] += v;
          }
        }
        double mean = 0.0;
        for (int32_t j = 0; j < k; ++j) mean += w[t * k + j] * dw[j];
        for (int32_t j = 0; j < k; ++j)
          dlt[idx[t * k + j]] = w[t * k + j] * (dw[j] - mean);
      }
    }
    free(buf);
  }
  return err;
}

/* Weight gradients of one expert e: dWg_e, dWu_e [f][d] and dWd_e [d][f],
 * summed over every assignment routed to e. Rows of the outputs are split
 * over threads; each thread walks all of e's assignments (recomputing
 * them), so no reduction across threads is needed. */
int oracle_weight_grads(int64_t T, int32_t E, int32_t k, int32_t d, int32_t f,
                        int32_t e, const int32_t *idx, const double *w,
                        const float *x, const float *Wg, const float *Wu,
                        const float *Wd, const float *dy, double *dWg,
                        double *dWu, double *dWd) {
  if (T < 1 || E < 1 || k < 1 || d < 1 || f < 1 || e < 0 || e >= E || !idx ||
      !w || !x || !Wg || !Wu || !Wd || !dy || !dWg || !dWu || !dWd)
    return OR_ERR_ARG;
  const int64_t TK = T * k;
  int64_t n = 0;
  for (int64_t a = 0; a < TK; ++a) n += idx[a] == e;
  int64_t *list = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  /* per assignment of e: dO (d), h, dg, du (f), x row (d), kept in fp64 */
  double *keep = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) *
                                  (size_t)(2 * d + 3 * f));
  if (!list || !keep) {
    free(list);
    free(keep);
    return OR_ERR_NOMEM;
  }
  n = 0;
  for (int64_t a = 0; a < TK; ++a)
    if (idx[a] == e) list[n++] = a;
  const int64_t wo = (int64_t)e * f * d;
  const int64_t stride = 2 * (int64_t)d + 3 * (int64_t)f;
  int err = OR_OK;
#pragma omp parallel
  {
    double *buf = (double *)malloc(sizeof(double) * (size_t)(4 * f + d));
    if (!buf) {
#pragma omp atomic write
      err = OR_ERR_NOMEM;
    } else {
      double *g = buf, *u = g + f, *a = u + f, *o = a + f;
#pragma omp for schedule(static)
      for (int64_t s = 0; s < n; ++s) {
        const int64_t asg = list[s];
        const int64_t t = asg / k;
        double *kp = keep + s * stride;
        double *xr = kp, *dO = xr + d, *h = dO + d, *dg = h + f, *du = dg + f;
        for (int32_t i = 0; i < d; ++i) xr[i] = (double)x[t * d + i];
        expert_recompute(d, f, xr, Wg + wo, Wu + wo, Wd + wo, g, u, a, h, o);
        for (int32_t m = 0; m < d; ++m) dO[m] = w[asg] * (double)dy[t * d + m];
        expert_dgate(d, f, dO, Wd + wo, g, u, a, dg, du);
      }
    }
    free(buf);
  }
  if (err == OR_OK) {
    /* sums over e's assignments in ascending assignment order */
#pragma omp parallel for schedule(static)
    for (int32_t q = 0; q < f; ++q) {
      for (int32_t i = 0; i < d; ++i) {
        double sg = 0.0, su = 0.0;
        for (int64_t s = 0; s < n; ++s) {
          const double *kp = keep + s * stride;
          sg += kp[2 * d + f + q] * kp[i];
          su += kp[2 * d + 2 * f + q] * kp[i];
        }
        dWg[(int64_t)q * d + i] = sg;
        dWu[(int64_t)q * d + i] = su;
      }
    }
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < d; ++m) {
      for (int32_t q = 0; q < f; ++q) {
        double sd = 0.0;
        for (int64_t s = 0; s < n; ++s) {
          const double *kp = keep + s * stride;
          sd += kp[d + m] * kp[2 * d + q];
        }
        dWd[(int64_t)m * f + q] = sd;
      }
    }
  }
  free(list);
  free(keep);
  return err;
}
