/*
 * sanitize_driver.c -- exercises every entry point of mlora_oracle.c on small
 * inputs, the error paths included, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py). Test
 * infrastructure only. Exits 0 when every call returns the expected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int mlo_segment(int, const int32_t*, int, int32_t*, int32_t*, int32_t*);
int mlo_check_meta(int, int, const int32_t*, const int32_t*, const int32_t*, const int32_t*, int,
                   const int32_t*);
int mlo_token_map(int, int, const int32_t*, const int32_t*, int32_t*, int32_t*);
int mlo_linear(int, int, int, const float*, const float*, int, const int32_t*, const int64_t*,
               const int64_t*, const float*, const float*, int, const int32_t*, const int32_t*,
               const int32_t*, const float*, const int32_t*, int, int, const int32_t*, double*, double*,
               int);
int mlo_merge(int, int, int, const float*, const float*, const float*, double, double*, int);

static int fails = 0;
static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
    ++fails;
  }
}

int main(void) {
  enum { T = 7, D_IN = 12, D_OUT = 9, CAP = 3 };
  float x[T * D_IN], W[D_OUT * D_IN], A[(2 + 3) * D_IN], B[D_OUT * (2 + 3)];
  for (int i = 0; i < T * D_IN; ++i) x[i] = (float)((i * 37) % 11) - 5.0f;
  for (int i = 0; i < D_OUT * D_IN; ++i) W[i] = (float)((i * 13) % 7) * 0.25f;
  for (int i = 0; i < 5 * D_IN; ++i) A[i] = (float)((i * 5) % 9) * 0.125f;
  for (int i = 0; i < D_OUT * 5; ++i) B[i] = (float)((i * 3) % 5) * 0.5f;
  /* adapters 0 (rank 2) and 2 (rank 3); slot 1 empty */
  const int32_t rank[CAP] = {2, 0, 3};
  const int64_t a_off[CAP] = {0, 0, 2 * D_IN};
  const int64_t b_off[CAP] = {0, 0, D_OUT * 2};

  /* canonical segmentation of unsorted ids, token map, checks */
  const int32_t ids[T] = {2, -1, 0, 2, 0, -1, 2};
  int32_t ti[T], ss[T + 2], sa[T + 1], ts[T], ta[T];
  const int S = mlo_segment(T, ids, CAP, ti, ss, sa);
  expect("segment count", S, 3);
  int32_t sr[T + 1];
  float sc[T + 1];
  for (int s = 0; s < S; ++s) {
    sr[s] = sa[s] >= 0 ? rank[sa[s]] : 0;
    sc[s] = 1.5f;
  }
  expect("token map", mlo_token_map(T, S, ss, sa, ts, ta), 0);
  expect("check meta", mlo_check_meta(T, S, ss, sa, sr, ti, CAP, rank), 0);
  const int32_t bad_ids[2] = {0, 5};
  int32_t ti2[2], ss2[4], sa2[3];
  expect("segment: id out of range", mlo_segment(2, bad_ids, CAP, ti2, ss2, sa2), -3);

  /* the layer, all rows and a row subset, LoRA-on and off */
  double y[T * D_OUT], yb[T * D_OUT];
  expect("linear", mlo_linear(T, D_IN, D_OUT, x, W, CAP, rank, a_off, b_off, A, B, S, ss, sa, sr, sc, ti, 1, T,
                              NULL, y, yb, 2), 0);
  const int32_t rows[3] = {6, 0, 3};
  expect("linear rows", mlo_linear(T, D_IN, D_OUT, x, W, CAP, rank, a_off, b_off, A, B, S, ss, sa, sr, sc, ti, 1,
                                   3, rows, y, NULL, 1), 0);
  expect("linear off", mlo_linear(T, D_IN, D_OUT, x, W, CAP, rank, a_off, b_off, A, B, 0, NULL, NULL, NULL,
                                  NULL, NULL, 0, T, NULL, y, NULL, 1), 0);
  /* error paths: unregistered adapter, rank mismatch, bad row, bad flag */
  int32_t sa_bad[T + 1], sr_bad[T + 1];
  for (int s = 0; s < S; ++s) { sa_bad[s] = sa[s] == 0 ? 1 : sa[s]; sr_bad[s] = sr[s] + (sa[s] == 2); }
  expect("linear: empty slot", mlo_linear(T, D_IN, D_OUT, x, W, CAP, rank, a_off, b_off, A, B, S, ss, sa_bad, NULL,
                                          sc, ti, 1, T, NULL, y, NULL, 1), -3);
  expect("linear: rank mismatch", mlo_linear(T, D_IN, D_OUT, x, W, CAP, rank, a_off, b_off, A, B, S, ss, sa,
                                             sr_bad, sc, ti, 1, T, NULL, y, NULL, 1), -4);
  const int32_t bad_row[1] = {T};
  expect("linear: row out of range", mlo_linear(T, D_IN, D_OUT, x, W, CAP, rank, a_off, b_off, A, B, S, ss, sa,
                                                sr, sc, ti, 1, 1, bad_row, y, NULL, 1), -1);
  expect("linear: lora_on 2", mlo_linear(T, D_IN, D_OUT, x, W, CAP, rank, a_off, b_off, A, B, S, ss, sa, sr, sc,
                                         ti, 2, T, NULL, y, NULL, 1), -1);

  /* merged weight, and its argument errors */
  double Wm[D_OUT * D_IN];
  expect("merge", mlo_merge(D_IN, D_OUT, 3, W, A + 2 * D_IN, B + D_OUT * 2, -0.5, Wm, 2), 0);
  expect("merge: rank 0", mlo_merge(D_IN, D_OUT, 0, W, NULL, NULL, 1.0, Wm, 1), 0);
  expect("merge: bad size", mlo_merge(0, D_OUT, 1, W, A, B, 1.0, Wm, 1), -1);

  if (fails) return 1;
  printf("sanitize driver: all oracle calls returned the expected status\n");
  return 0;
}
