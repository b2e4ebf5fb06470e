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
 * FP8 candidate table (quantised rows; the functions at the end of this
 * file). The draft may read its candidate rows in an 8-bit format instead of
 * bfloat16, halving the bytes that dominate the call. (Same section of the
 * tuning log: the upstream work on this bottleneck stores the candidate rows
 * in a low-precision float format and reports a further gain over bf16
 * rows.) Format: OCP 8-bit float E4M3 ("E4M3FN"): sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; no
 * infinities; S.1111.111 is NaN; the largest finite magnitude is 448. Each
 * row carries one scale 2^e, the smallest power of two with
 * max_j |w[j]| <= 448 * 2^e (e = 0 for an all-zero row), and stores element
 * j as the E4M3 value nearest to w[j] * 2^-e (ties to the even code). A
 * row's logit is 2^e * sum_j x[j] * value(q[j]), summed as above in double.
 *
 * MXFP4 candidate table (4-bit rows; the last functions of this file). The
 * same section names 4-bit float candidate rows for the upstream work; the
 * pages fix no block size or scale format, and the format taken here is the
 * OCP microscaling one, MXFP4: elements E2M1 (sign, 2 exponent bits with
 * bias 1, 1 mantissa bit; exponent field 0 holds 0 and 0.5; magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN), one E8M0 scale 2^e per
 * block of 32 consecutive elements of a row (code e + 127). The scale follows
 * the OCP MX rule: e = floor(log2(max |w| over the block)) - 2, clamped to
 * [-127, 127], e = -127 for an all-zero block; element j is the E2M1 value
 * nearest to w[j] * 2^-e (ties to the even code, magnitudes past 6 saturate
 * to 6; a negative value keeps its sign bit even when it rounds to zero).
 * Two codes share a byte, element 2i in the low nibble. A row's logit is
 * sum_j x[j] * 2^e(j / 32) * value(q[j]), summed as above in double.
 * A second scale reading (the "fit" rule) is offered beside the OCP one: the
 * smallest e with max |w| <= 6 * 2^e, so that no element of the block
 * saturates; same clamp, same zero block, same elements otherwise. It
 * differs from the OCP rule only in blocks whose largest magnitude lies
 * above 6 * 2^(floor(log2 max) - 2), where it takes e one larger.
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
/* The argmax decision over one query row's N double logits z: the first
 * maximum of the fp32-rounded logits, and the double runner-up among the
 * other rows (see mtp_oracle_argmax). */
static int decide_row(const double *z, int64_t N, const int32_t *ids, int32_t *top_id,
                      float *top_logit, double *top_exact, int32_t *runner_id,
                      double *runner_exact) {
  int64_t best = -1;
  float best_f = 0.0f;
  for (int64_t n = 0; n < N; ++n) {
    if (!isfinite(z[n])) return ORC_NOT_FINITE;
    float f = (float)z[n];
    if (best < 0 || f > best_f) { best = n; best_f = f; }
  }
  int64_t second = -1;
  double second_z = -INFINITY;
  for (int64_t n = 0; n < N; ++n) {
    if (n == best) continue;
    if (second < 0 || z[n] > second_z) { second = n; second_z = z[n]; }
  }
  *top_id = ids ? ids[best] : (int32_t)best;
  *top_logit = best_f;
  *top_exact = z[best];
  *runner_id = second < 0 ? -1 : (ids ? ids[second] : (int32_t)second);
  *runner_exact = second_z;
  return ORC_OK;
}

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
    rc = decide_row(z, N, ids, top_id + m, top_logit + m, top_exact + m, runner_id + m,
                    runner_exact + m);
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

/* ---- FP8 (E4M3) candidate table ---------------------------------------- */

/* The value of an E4M3 code (NaN for S.1111.111). */
double mtp_oracle_e4m3_value(uint8_t code) {
  const int e = (code >> 3) & 15;
  const int m = code & 7;
  if (e == 15 && m == 7) return NAN;
  /* subnormal: m * 2^-9; normal: (1 + m/8) * 2^(e-7) = (8 + m) * 2^(e-10) */
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (code & 0x80) ? -v : v;
}

/* The E4M3 code nearest to x (ties to the even code, i.e. mantissa bit 0
 * clear); magnitudes beyond 448 saturate to +-448; NaN gives 0x7F. */
uint8_t mtp_oracle_e4m3_round(double x) {
  if (isnan(x)) return 0x7F;
  const uint8_t s = signbit(x) ? 0x80 : 0x00;
  const double a = fabs(x);
  if (a >= 448.0) return s | 0x7E;
  if (a < ldexp(1.0, -6)) {
    /* subnormal spacing 2^-9: round a / 2^-9 to an integer, ties to even;
       8 is the smallest normal, whose code is also 8 */
    const double r = nearbyint(ldexp(a, 9));
    return s | (uint8_t)r;
  }
  int E;
  frexp(a, &E);                    /* a = f * 2^E, f in [0.5, 1) */
  int ue = E - 1;                  /* a in [2^ue, 2^(ue+1)) */
  double r = nearbyint(ldexp(a, 3 - ue));  /* 8..16: 1.mmm in eighths */
  if (r == 16.0) { r = 8.0; ue += 1; }
  if (ue > 8 || (ue == 8 && r > 14.0)) return s | 0x7E;
  return s | (uint8_t)(((ue + 7) << 3) | ((int)r - 8));
}

int mtp_oracle_e4m3_round_array(const double *x, int64_t n, uint8_t *out) {
  if (!x || !out || n < 0) return ORC_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = mtp_oracle_e4m3_round(x[i]);
  return ORC_OK;
}

/* The row's scale exponent: the smallest e with max|w| <= 448 * 2^e (0 for
 * an all-zero row). */
int mtp_oracle_fp8_row_exponent(const uint16_t *w, int64_t H, int32_t *e_out) {
  if (!w || !e_out || H <= 0) return ORC_BAD_ARG;
  double amax = 0.0;
  for (int64_t j = 0; j < H; ++j) {
    const double v = fabs(bf16_to_double(w[j]));
    if (!isfinite(v)) return ORC_NOT_FINITE;
    if (v > amax) amax = v;
  }
  if (amax == 0.0) { *e_out = 0; return ORC_OK; }
  int e = ilogb(amax) - 8;
  while (ldexp(448.0, e) < amax) ++e;
  while (ldexp(448.0, e - 1) >= amax) --e;
  *e_out = e;
  return ORC_OK;
}

/* Quantise the candidate rows head[ids[i]] (ids NULL: rows 0..C-1):
 * q[i][j] = E4M3(head[ids[i]][j] * 2^-e[i]), exps[i] = e[i]. */
int mtp_oracle_quantize_fp8(const uint16_t *head, int64_t V, int64_t H, const int32_t *ids,
                            int64_t C, uint8_t *q, int32_t *exps) {
  if (!head || !q || !exps || V <= 0 || H <= 0 || C <= 0) return ORC_BAD_ARG;
  if (ids && mtp_oracle_check_ids(ids, C, V) != ORC_OK) return ORC_BAD_IDS;
  if (!ids && C > V) return ORC_BAD_ARG;
  int rc = ORC_OK;
  for (int64_t i = 0; i < C; ++i) {
    const uint16_t *w = head + (int64_t)(ids ? ids[i] : i) * H;
    int32_t e = 0;
    const int r = mtp_oracle_fp8_row_exponent(w, H, &e);
    if (r != ORC_OK) { rc = r; break; }
    exps[i] = e;
    for (int64_t j = 0; j < H; ++j) q[i * H + j] = mtp_oracle_e4m3_round(ldexp(bf16_to_double(w[j]), -e));
  }
  return rc;
}

/* One fp8 row's logit: 2^e * sum over j of x[j] * value(q[j]), in order,
 * in double (each product is exact). */
static double dot_fp8(const uint16_t *x, const uint8_t *q, int32_t e, int64_t H) {
  double s = 0.0;
  for (int64_t j = 0; j < H; ++j) s += bf16_to_double(x[j]) * mtp_oracle_e4m3_value(q[j]);
  return ldexp(s, e);
}

/* Argmax of every query row over an fp8 table of N rows (as
 * mtp_oracle_argmax, with each row's logit from dot_fp8). */
int mtp_oracle_fp8_argmax(const uint16_t *x, int64_t M, const uint8_t *q, const int32_t *exps,
                          const int32_t *ids, int64_t N, int64_t H, int32_t *top_id,
                          float *top_logit, double *top_exact, int32_t *runner_id,
                          double *runner_exact) {
  if (!x || !q || !exps || !top_id || !top_logit || !top_exact || !runner_id || !runner_exact ||
      M < 0 || N <= 0 || H <= 0)
    return ORC_BAD_ARG;
  double *z = (double *)malloc((size_t)N * sizeof(double));
  if (!z) return ORC_NO_MEMORY;
  int rc = ORC_OK;
  for (int64_t m = 0; m < M && rc == ORC_OK; ++m) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) z[n] = dot_fp8(x + m * H, q + n * H, exps[n], H);
    rc = decide_row(z, N, ids, top_id + m, top_logit + m, top_exact + m, runner_id + m,
                    runner_exact + m);
  }
  free(z);
  return rc;
}

/* ---- MXFP4 candidate table ---------------------------------------------- */

/* The value of an E2M1 code (low 4 bits). */
double mtp_oracle_e2m1_value(uint8_t code) {
  const int e = (code >> 1) & 3;
  const int m = code & 1;
  /* exponent 0: m * 0.5; otherwise (1 + m/2) * 2^(e-1) = (2 + m) * 2^(e-2) */
  const double v = e == 0 ? 0.5 * m : ldexp((double)(2 + m), e - 2);
  return (code & 8) ? -v : v;
}

/* The E2M1 code nearest to x (ties to the even code, i.e. mantissa bit 0
 * clear); magnitudes beyond 6 saturate to 6; x < 0 sets the sign bit. */
uint8_t mtp_oracle_e2m1_round(double x) {
  const uint8_t s = x < 0.0 ? 8 : 0;
  const double a = fabs(x);
  if (!(a < 6.0)) return s | 7;                 /* also NaN (out of contract) */
  if (a < 1.0) {
    /* spacing 0.5: round 2a to an integer, ties to even; 2 is the code of 1.0 */
    return s | (uint8_t)nearbyint(2.0 * a);
  }
  int E;
  frexp(a, &E);                                 /* a = f * 2^E, f in [0.5, 1) */
  int ue = E - 1;                               /* a in [2^ue, 2^(ue+1)), ue 0..2 */
  double r = nearbyint(ldexp(a, 1 - ue));       /* 2 or 3 in halves of 2^ue; 4: next binade */
  if (r == 4.0) { r = 2.0; ue += 1; }
  return s | (uint8_t)(((ue + 1) << 1) | ((int)r - 2));
}

int mtp_oracle_e2m1_round_array(const double *x, int64_t n, uint8_t *out) {
  if (!x || !out || n < 0) return ORC_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = mtp_oracle_e2m1_round(x[i]);
  return ORC_OK;
}

/* A block's scale exponent: floor(log2(max |w|)) - 2, clamped to [-127, 127];
 * -127 for an all-zero block. */
int mtp_oracle_mx_block_exponent(const uint16_t *w, int64_t n, int32_t *e_out) {
  if (!w || !e_out || n <= 0) return ORC_BAD_ARG;
  double amax = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double v = fabs(bf16_to_double(w[j]));
    if (!isfinite(v)) return ORC_NOT_FINITE;
    if (v > amax) amax = v;
  }
  int e = amax == 0.0 ? -127 : ilogb(amax) - 2;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  *e_out = e;
  return ORC_OK;
}

/* A block's scale exponent under the fit rule: the smallest e with
 * max |w| <= 6 * 2^e, clamped to [-127, 127]; -127 for an all-zero block.
 * 6 * 2^(ilogb(max) - 3) < 2^ilogb(max) <= max, so the search starts below
 * the answer and steps up to it. */
int mtp_oracle_mx_block_exponent_fit(const uint16_t *w, int64_t n, int32_t *e_out) {
  if (!w || !e_out || n <= 0) return ORC_BAD_ARG;
  double amax = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double v = fabs(bf16_to_double(w[j]));
    if (!isfinite(v)) return ORC_NOT_FINITE;
    if (v > amax) amax = v;
  }
  int e = -127;
  if (amax != 0.0) {
    e = ilogb(amax) - 3;
    while (ldexp(6.0, e) < amax) ++e;
  }
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  *e_out = e;
  return ORC_OK;
}

/* Quantise the candidate rows head[ids[i]] (ids NULL: rows 0..C-1) to MXFP4:
 * q[i][j / 2] holds the codes of elements j (low nibble, j even) and j + 1;
 * scales[i][b] = e + 127 of block b (elements 32b .. 32b + 31). H % 32 == 0.
 * rule 0: the OCP scale rule; rule 1: the fit rule. */
int mtp_oracle_quantize_mxfp4_rule(const uint16_t *head, int64_t V, int64_t H,
                                   const int32_t *ids, int64_t C, uint8_t *q, uint8_t *scales,
                                   int rule) {
  if (rule != 0 && rule != 1) return ORC_BAD_ARG;
  if (!head || !q || !scales || V <= 0 || H <= 0 || H % 32 != 0 || C <= 0) return ORC_BAD_ARG;
  if (ids && mtp_oracle_check_ids(ids, C, V) != ORC_OK) return ORC_BAD_IDS;
  if (!ids && C > V) return ORC_BAD_ARG;
  const int64_t nb = H / 32;
  for (int64_t i = 0; i < C; ++i) {
    const uint16_t *w = head + (int64_t)(ids ? ids[i] : i) * H;
    for (int64_t b = 0; b < nb; ++b) {
      int32_t e = 0;
      const int r = rule == 0 ? mtp_oracle_mx_block_exponent(w + 32 * b, 32, &e)
                              : mtp_oracle_mx_block_exponent_fit(w + 32 * b, 32, &e);
      if (r != ORC_OK) return r;
      scales[i * nb + b] = (uint8_t)(e + 127);
      for (int64_t j = 32 * b; j < 32 * b + 32; j += 2) {
        const uint8_t lo = mtp_oracle_e2m1_round(ldexp(bf16_to_double(w[j]), -e));
        const uint8_t hi = mtp_oracle_e2m1_round(ldexp(bf16_to_double(w[j + 1]), -e));
        q[i * (H / 2) + j / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
  return ORC_OK;
}

int mtp_oracle_quantize_mxfp4(const uint16_t *head, int64_t V, int64_t H, const int32_t *ids,
                              int64_t C, uint8_t *q, uint8_t *scales) {
  return mtp_oracle_quantize_mxfp4_rule(head, V, H, ids, C, q, scales, 0);
}

/* One MXFP4 row's logit: sum over j of x[j] * 2^e(j / 32) * value(q[j]), in
 * order, in double (each term is exact). */
static double dot_mxfp4(const uint16_t *x, const uint8_t *q, const uint8_t *scales, int64_t H) {
  double s = 0.0;
  for (int64_t j = 0; j < H; ++j) {
    const uint8_t code = (j & 1) ? (q[j / 2] >> 4) : (q[j / 2] & 15);
    const int e = (int)scales[j / 32] - 127;
    s += bf16_to_double(x[j]) * ldexp(mtp_oracle_e2m1_value(code), e);
  }
  return s;
}

/* Argmax of every query row over an MXFP4 table of N rows (as
 * mtp_oracle_argmax, with each row's logit from dot_mxfp4). */
int mtp_oracle_mxfp4_argmax(const uint16_t *x, int64_t M, const uint8_t *q,
                            const uint8_t *scales, const int32_t *ids, int64_t N, int64_t H,
                            int32_t *top_id, float *top_logit, double *top_exact,
                            int32_t *runner_id, double *runner_exact) {
  if (!x || !q || !scales || !top_id || !top_logit || !top_exact || !runner_id ||
      !runner_exact || M < 0 || N <= 0 || H <= 0 || H % 32 != 0)
    return ORC_BAD_ARG;
  double *z = (double *)malloc((size_t)N * sizeof(double));
  if (!z) return ORC_NO_MEMORY;
  int rc = ORC_OK;
  for (int64_t m = 0; m < M && rc == ORC_OK; ++m) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
      z[n] = dot_mxfp4(x + m * H, q + n * (H / 2), scales + n * (H / 32), H);
    rc = decide_row(z, N, ids, top_id + m, top_logit + m, top_exact + m, runner_id + m,
                    runner_exact + m);
  }
  free(z);
  return rc;
}
