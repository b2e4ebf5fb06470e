/*
 * CPU oracle for the MTP draft / verify LM-head path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline of the benchmark can compare the GPU kernels with a plain, slow,
 * obviously correct statement of what they compute. It shares no code with
 * the HIP library.
 *
 * What is computed, and where it is defined:
 *   - Draft step: score the MTP hidden state against a reduced candidate
 *     table, take the highest-scoring row and report its global token id.
 *     (Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big
 *     table" (少读一张大表): each rank searches its own candidate rows for the
 *     maximum and exchanges the maximum score with its global token id.)
 *   - Verify step: score the k+1 verify positions against the full head and
 *     take each position's argmax (same section: the main model keeps
 *     verifying with the full vocabulary).
 *   - Acceptance: keep the drafts while they agree with the target's argmax;
 *     at the first disagreement (or after all k) emit the target's own token.
 *     (Edge-inference runtime blog, section 2.1: speculative use of the MTP
 *     head accepts more tokens than steps executed; long-context blog,
 *     section 5: MTP proposal -> target verification -> accept some tokens.)
 *
 * Arithmetic. Inputs are bfloat16 bit patterns (uint16). Each element is
 * widened exactly to double, products are exact in double, and each logit
 * is one sequential double-precision sum over the hidden index j = 0..H-1.
 * Its error is below H * 2^-53 * sum|terms|, far under fp32 resolution.
 * Where a floating-point value decides an integer (the argmax), the decision
 * is taken in fp32, the precision the GPU kernels accumulate in: every
 * logit is rounded once to float and the first (lowest index) maximum wins.
 * Threads split the list of table rows only; each logit's arithmetic does
 * not depend on the thread count.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
  ORC_OK = 0,
  ORC_BAD_ARG = 1,
  ORC_BAD_IDS = 4,
  ORC_NO_MEMORY = 6,
  ORC_NOT_FINITE = 7
};

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* One logit: sum over j of x[j] * w[j], in order, in double. */
static double dot_bf16(const uint16_t *x, const uint16_t *w, int64_t H) {
  double s = 0.0;
  for (int64_t j = 0; j < H; ++j) s += bf16_to_double(x[j]) * bf16_to_double(w[j]);
  return s;
}

int mtp_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* z[m*N + n] = dot(x[m], w[n]) for m < M, n < N. */
int mtp_oracle_logits(const uint16_t *x, int64_t M, const uint16_t *w, int64_t N, int64_t H,
                      double *z) {
  if (!x || !w || !z || M < 0 || N < 0 || H <= 0) return ORC_BAD_ARG;
  for (int64_t m = 0; m < M; ++m) {
    const uint16_t *xm = x + m * H;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) z[m * N + n] = dot_bf16(xm, w + n * H, H);
  }
  return ORC_OK;
}

/* Logits of selected (row, table row) pairs: z[i] = dot(x[rows[i]], w[cols[i]]). */
int mtp_oracle_pair_logits(const uint16_t *x, const uint16_t *w, int64_t H, const int64_t *rows,
                           const int64_t *cols, int64_t n_pairs, double *z) {
  if (!x || !w || !rows || !cols || !z || H <= 0 || n_pairs < 0) return ORC_BAD_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_pairs; ++i) z[i] = dot_bf16(x + rows[i] * H, w + cols[i] * H, H);
  return ORC_OK;
}

/*
 * Argmax of every query row over N table rows.
 *   ids: global token id of each table row (NULL: row index is the id).
 * Per query row m:
 *   top_id[m], top_logit[m]  token id and fp32 logit of the first row whose
 *                            fp32-rounded logit is maximal;
 *   top_exact[m]             that row's double logit;
 *   runner_id[m], runner_exact[m]
 *                            the largest double logit among the other rows
 *                            (first such row), used to find near-ties; -1 and
 *                            -inf if N == 1.
 */
int mtp_oracle_argmax(const uint16_t *x, int64_t M, const uint16_t *w, const int32_t *ids,
                      int64_t N, int64_t H, int32_t *top_id, float *top_logit,
                      double *top_exact, int32_t *runner_id, double *runner_exact) {
  if (!x || !w || !top_id || !top_logit || !top_exact || !runner_id || !runner_exact || M < 0 ||
      N <= 0 || H <= 0)
    return ORC_BAD_ARG;
  double *z = (double *)malloc((size_t)N * sizeof(double));
  if (!z) return ORC_NO_MEMORY;
  int rc = ORC_OK;
  for (int64_t m = 0; m < M && rc == ORC_OK; ++m) {
    mtp_oracle_logits(x + m * H, 1, w, N, H, z);
    /* fp32 decision: first maximum of the rounded logits. */
    int64_t best = -1;
    float best_f = 0.0f;
    for (int64_t n = 0; n < N; ++n) {
      if (!isfinite(z[n])) { rc = ORC_NOT_FINITE; break; }
      float f = (float)z[n];
      if (best < 0 || f > best_f) { best = n; best_f = f; }
    }
    if (rc != ORC_OK) break;
    /* runner-up in double over the other rows */
    int64_t second = -1;
    double second_z = -INFINITY;
    for (int64_t n = 0; n < N; ++n) {
      if (n == best) continue;
      if (second < 0 || z[n] > second_z) { second = n; second_z = z[n]; }
    }
    top_id[m] = ids ? ids[best] : (int32_t)best;
    top_logit[m] = best_f;
    top_exact[m] = z[best];
    runner_id[m] = second < 0 ? -1 : (ids ? ids[second] : (int32_t)second);
    runner_exact[m] = second_z;
  }
  free(z);
  return rc;
}

/*
 * Greedy acceptance for B sequences with k drafts each.
 *   draft [B][k], target [B][k+1] (target argmax at verify positions 0..k).
 *   n_accept[b] = first p < k with draft[b][p] != target[b][p], else k.
 *   tokens[b][0..n_accept[b]] = target[b][0..n_accept[b]] (the accepted
 *   drafts, which equal the target there, followed by the target's token at
 *   the stopping position), remaining slots -1.
 */
int mtp_oracle_accept(const int32_t *draft, const int32_t *target, int64_t B, int64_t k,
                      int32_t *n_accept, int32_t *tokens) {
  if (B < 0 || k < 0 || !target || !n_accept || !tokens || (k > 0 && !draft)) return ORC_BAD_ARG;
  for (int64_t b = 0; b < B; ++b) {
    int64_t n = 0;
    while (n < k && draft[b * k + n] == target[b * (k + 1) + n]) ++n;
    n_accept[b] = (int32_t)n;
    for (int64_t p = 0; p <= k; ++p)
      tokens[b * (k + 1) + p] = p <= n ? target[b * (k + 1) + p] : -1;
  }
  return ORC_OK;
}

/* Candidate ids must be strictly ascending and inside [0, V). */
int mtp_oracle_check_ids(const int32_t *ids, int64_t C, int64_t V) {
  if (!ids || C <= 0 || V <= 0) return ORC_BAD_ARG;
  for (int64_t i = 0; i < C; ++i) {
    if (ids[i] < 0 || ids[i] >= V) return ORC_BAD_IDS;
    if (i > 0 && ids[i] <= ids[i - 1]) return ORC_BAD_IDS;
  }
  return ORC_OK;
}

/* table[i][:] = head[ids[i]][:] (the packed candidate sub-table). */
int mtp_oracle_pack(const uint16_t *head, int64_t V, int64_t H, const int32_t *ids, int64_t C,
                    uint16_t *table) {
  if (!head || !table || H <= 0) return ORC_BAD_ARG;
  int rc = mtp_oracle_check_ids(ids, C, V);
  if (rc != ORC_OK) return rc;
  for (int64_t i = 0; i < C; ++i)
    memcpy(table + i * H, head + (int64_t)ids[i] * H, (size_t)H * sizeof(uint16_t));
  return ORC_OK;
}
