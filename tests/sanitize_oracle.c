/*
 * Host driver for the sanitizer build of the CPU oracle (test infrastructure).
 * Built together with oracle/mtp_oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (no OpenMP, so every loop runs in this thread),
 * it calls every exported oracle function on small seeded inputs, at the edge
 * shapes (one row, one column block, k = 0, B = 0, all-zero rows, extreme
 * codes) and on the argument errors, and checks the status codes. Any memory
 * or undefined-behaviour error aborts the run with a report on stderr.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int mtp_oracle_threads(void);
int mtp_oracle_logits(const uint16_t *x, int64_t M, const uint16_t *w, int64_t N, int64_t H,
                      double *z);
int mtp_oracle_pair_logits(const uint16_t *x, const uint16_t *w, int64_t H, const int64_t *rows,
                           const int64_t *cols, int64_t n_pairs, double *z);
int mtp_oracle_argmax(const uint16_t *x, int64_t M, const uint16_t *w, const int32_t *ids,
                      int64_t N, int64_t H, int32_t *top_id, float *top_logit,
                      double *top_exact, int32_t *runner_id, double *runner_exact);
int mtp_oracle_accept(const int32_t *draft, const int32_t *target, int64_t B, int64_t k,
                      int32_t *n_accept, int32_t *tokens);
int mtp_oracle_check_ids(const int32_t *ids, int64_t C, int64_t V);
int mtp_oracle_pack(const uint16_t *head, int64_t V, int64_t H, const int32_t *ids, int64_t C,
                    uint16_t *table);
double mtp_oracle_e4m3_value(uint8_t code);
uint8_t mtp_oracle_e4m3_round(double x);
int mtp_oracle_e4m3_round_array(const double *x, int64_t n, uint8_t *out);
int mtp_oracle_fp8_row_exponent(const uint16_t *w, int64_t H, int32_t *e_out);
int mtp_oracle_quantize_fp8(const uint16_t *head, int64_t V, int64_t H, const int32_t *ids,
                            int64_t C, uint8_t *q, int32_t *exps);
int mtp_oracle_fp8_argmax(const uint16_t *x, int64_t M, const uint8_t *q, const int32_t *exps,
                          const int32_t *ids, int64_t N, int64_t H, int32_t *top_id,
                          float *top_logit, double *top_exact, int32_t *runner_id,
                          double *runner_exact);
double mtp_oracle_e2m1_value(uint8_t code);
uint8_t mtp_oracle_e2m1_round(double x);
int mtp_oracle_e2m1_round_array(const double *x, int64_t n, uint8_t *out);
int mtp_oracle_mx_block_exponent(const uint16_t *w, int64_t n, int32_t *e_out);
int mtp_oracle_quantize_mxfp4(const uint16_t *head, int64_t V, int64_t H, const int32_t *ids,
                              int64_t C, uint8_t *q, uint8_t *scales);
int mtp_oracle_mx_block_exponent_fit(const uint16_t *w, int64_t n, int32_t *e_out);
int mtp_oracle_quantize_mxfp4_rule(const uint16_t *head, int64_t V, int64_t H,
                                   const int32_t *ids, int64_t C, uint8_t *q, uint8_t *scales,
                                   int rule);
int mtp_oracle_mxfp4_argmax(const uint16_t *x, int64_t M, const uint8_t *q,
                            const uint8_t *scales, const int32_t *ids, int64_t N, int64_t H,
                            int32_t *top_id, float *top_logit, double *top_exact,
                            int32_t *runner_id, double *runner_exact);

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (uint32_t)(rng_state >> 16);
}
/* A finite bfloat16 with magnitude in [2^-9, 2^3). */
static uint16_t rand_bf16(void) {
  const uint32_t r = next_u32();
  const uint32_t exp = 118u + (r % 12u);
  return (uint16_t)(((r >> 8) & 1u) << 15 | exp << 7 | ((r >> 9) & 0x7Fu));
}

/* Runs every function once per shape: M query rows, N table rows, H columns,
 * with a head of V rows from which C candidate rows are picked. */
static void run_shape(int64_t M, int64_t V, int64_t C, int64_t H) {
  uint16_t *head = malloc((size_t)(V * H) * sizeof *head);
  uint16_t *x = malloc((size_t)(M * H) * sizeof *x);
  uint16_t *table = malloc((size_t)(C * H) * sizeof *table);
  int32_t *ids = malloc((size_t)C * sizeof *ids);
  double *z = malloc((size_t)(M * V) * sizeof *z);
  int32_t *top = malloc((size_t)M * sizeof *top), *run = malloc((size_t)M * sizeof *run);
  float *topf = malloc((size_t)M * sizeof *topf);
  double *tope = malloc((size_t)M * sizeof *tope), *rune = malloc((size_t)M * sizeof *rune);
  for (int64_t i = 0; i < V * H; ++i) head[i] = rand_bf16();
  for (int64_t j = 0; j < H; ++j) head[j] = 0;  /* row 0: all zero */
  for (int64_t i = 0; i < M * H; ++i) x[i] = rand_bf16();
  /* ids: every (V / C)-th row, strictly ascending */
  for (int64_t i = 0; i < C; ++i) ids[i] = (int32_t)(i * (V / C));

  EXPECT(mtp_oracle_check_ids(ids, C, V) == 0);
  EXPECT(mtp_oracle_pack(head, V, H, ids, C, table) == 0);
  EXPECT(mtp_oracle_logits(x, M, head, V, H, z) == 0);
  EXPECT(mtp_oracle_argmax(x, M, table, ids, C, H, top, topf, tope, run, rune) == 0);
  EXPECT(mtp_oracle_argmax(x, M, head, NULL, V, H, top, topf, tope, run, rune) == 0);
  {
    int64_t rows[3] = {0, M - 1, M / 2}, cols[3] = {V - 1, 0, V / 2};
    double pz[3];
    EXPECT(mtp_oracle_pair_logits(x, head, H, rows, cols, 3, pz) == 0);
    EXPECT(pz[0] == z[0 * V + V - 1]);
  }
  {
    uint8_t *q8 = malloc((size_t)(C * H));
    int32_t *e8 = malloc((size_t)C * sizeof *e8);
    EXPECT(mtp_oracle_quantize_fp8(head, V, H, ids, C, q8, e8) == 0);
    EXPECT(mtp_oracle_quantize_fp8(head, V, H, NULL, C, q8, e8) == 0);
    EXPECT(mtp_oracle_fp8_argmax(x, M, q8, e8, ids, C, H, top, topf, tope, run, rune) == 0);
    free(q8);
    free(e8);
  }
  if (H % 32 == 0) {
    uint8_t *q4 = malloc((size_t)(C * H / 2));
    uint8_t *s4 = malloc((size_t)(C * H / 32));
    EXPECT(mtp_oracle_quantize_mxfp4(head, V, H, ids, C, q4, s4) == 0);
    EXPECT(mtp_oracle_quantize_mxfp4(head, V, H, NULL, C, q4, s4) == 0);
    EXPECT(mtp_oracle_quantize_mxfp4_rule(head, V, H, ids, C, q4, s4, 1) == 0);
    EXPECT(mtp_oracle_mxfp4_argmax(x, M, q4, s4, NULL, C, H, top, topf, tope, run, rune) == 0);
    free(q4);
    free(s4);
  }
  free(head); free(x); free(table); free(ids); free(z);
  free(top); free(run); free(topf); free(tope); free(rune);
}

int main(void) {
  EXPECT(mtp_oracle_threads() >= 1);
  /* shapes: single row and column block, ragged widths, several rows */
  run_shape(1, 1, 1, 32);
  run_shape(1, 7, 3, 8);
  run_shape(3, 64, 16, 96);
  run_shape(5, 130, 33, 256);
  run_shape(2, 300, 100, 40);

  /* acceptance: k = 0, B = 0, full and partial agreement */
  {
    int32_t target[2 * 4] = {5, 6, 7, 8, 1, 2, 3, 4};
    int32_t draft[2 * 3] = {5, 6, 7, 1, 9, 3};
    int32_t n[2], tok[2 * 4];
    EXPECT(mtp_oracle_accept(draft, target, 2, 3, n, tok) == 0);
    EXPECT(n[0] == 3 && tok[3] == 8 && n[1] == 1 && tok[5] == 2 && tok[6] == -1);
    EXPECT(mtp_oracle_accept(NULL, target, 2, 0, n, tok) == 0);
    EXPECT(n[0] == 0 && tok[0] == 5);
    EXPECT(mtp_oracle_accept(draft, target, 0, 3, n, tok) == 0);
  }
  /* element formats: every code, and rounding at the extremes */
  for (int c = 0; c < 256; ++c) {
    const double v = mtp_oracle_e4m3_value((uint8_t)c);
    if (isfinite(v)) EXPECT(mtp_oracle_e4m3_round(v) == (uint8_t)c || v == 0.0);
    const double f = mtp_oracle_e2m1_value((uint8_t)c);
    EXPECT(isfinite(f));
  }
  {
    const double xs[] = {0.0, -0.0, 1e-30, -1e-30, 448.0, 1e30, -1e30, 0.75, 1.75, 3.5, 6.5};
    const int64_t n = (int64_t)(sizeof xs / sizeof xs[0]);
    uint8_t out[16];
    EXPECT(mtp_oracle_e4m3_round_array(xs, n, out) == 0);
    EXPECT(mtp_oracle_e2m1_round_array(xs, n, out) == 0);
  }
  {
    uint16_t w[64];
    int32_t e = 0;
    memset(w, 0, sizeof w);
    EXPECT(mtp_oracle_fp8_row_exponent(w, 64, &e) == 0 && e == 0);
    EXPECT(mtp_oracle_mx_block_exponent(w, 32, &e) == 0 && e == -127);
    EXPECT(mtp_oracle_mx_block_exponent_fit(w, 32, &e) == 0 && e == -127);
    w[5] = 0x7F7F;  /* largest finite bfloat16 */
    EXPECT(mtp_oracle_fp8_row_exponent(w, 64, &e) == 0);
    EXPECT(mtp_oracle_mx_block_exponent(w, 32, &e) == 0 && e == 125);
    EXPECT(mtp_oracle_mx_block_exponent_fit(w, 32, &e) == 0 && e == 126);
    w[6] = 0x0001;  /* smallest subnormal bfloat16 */
    w[5] = 0;
    EXPECT(mtp_oracle_mx_block_exponent(w, 32, &e) == 0 && e == -127);
    EXPECT(mtp_oracle_mx_block_exponent_fit(w, 32, &e) == 0 && e == -127);
    w[7] = 0x7F80;  /* +inf: outside the contract, reported */
    EXPECT(mtp_oracle_fp8_row_exponent(w, 64, &e) == 7);
  }
  /* argument errors */
  {
    uint16_t h[8] = {0};
    int32_t bad_ids[3] = {2, 1, 0};
    uint16_t t[24];
    EXPECT(mtp_oracle_check_ids(bad_ids, 3, 4) == 4);
    EXPECT(mtp_oracle_pack(h, 1, 8, bad_ids, 3, t) == 4);
    EXPECT(mtp_oracle_logits(NULL, 1, h, 1, 8, NULL) == 1);
    EXPECT(mtp_oracle_argmax(h, 1, h, NULL, 0, 8, NULL, NULL, NULL, NULL, NULL) == 1);
    EXPECT(mtp_oracle_accept(NULL, NULL, 1, 1, NULL, NULL) == 1);
    EXPECT(mtp_oracle_quantize_mxfp4(h, 1, 8, NULL, 1, (uint8_t *)t, (uint8_t *)t) == 1);
    EXPECT(mtp_oracle_quantize_mxfp4_rule(h, 1, 32, NULL, 1, (uint8_t *)t, (uint8_t *)t, 2) == 1);
  }
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("sanitized oracle run ok\n");
  return 0;
}
