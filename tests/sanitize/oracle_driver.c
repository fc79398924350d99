/* The CPU oracle over small problems, their degenerate shapes and their
 * error cases, built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitize_cpu.py.  Exit status 0 when every call returned what it
 * should; the sanitizers abort on the first memory or UB error. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's entry points (oracle/oracle.c) */
int oracle_gemm_rs(int, int, int, int, int, int, int, const void*, const void*, void*, void*);
int oracle_gemm_rs_points(int, int, int, int, int, int, int, const void*, const void*, int64_t, const int64_t*,
                          const int64_t*, void*, void*);
int oracle_gemm_ar(int, int, int, int, int, int, int, const void*, const void*, void*, void*);
int oracle_gemm_a2a(int, int, int64_t, int, int, int, int, const void*, const void*, const int64_t*,
                    const int32_t*, const int32_t*, int64_t, void*);
int oracle_a2a_gemm(int, int, int, int, int, int, int, int, int, const void*, const int32_t*, const void*, int,
                    int64_t, void*, void*, int64_t*, int32_t*, int32_t*, int64_t*);
int oracle_gemv_ar(int, int, int, int, int, int, int, const void*, const void*, void*, void*);
int oracle_ag_gemm(int, int, int, int, int, int, const void* const*, const void*, void*, void*);
int oracle_ag_gemm_points(int, int, int, int, int, int, const void* const*, const void*, int64_t, const int64_t*,
                          const int64_t*, void*);
int oracle_embbag_a2a(int, int64_t, int, int, int, int, const float*, const int32_t*, const int64_t*, float*);

enum { F32 = 0, BF16 = 1 };
static int fails = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c);          \
      ++fails;                                                      \
    }                                                               \
  } while (0)

static uint64_t rng = 88172645463325252ull;
static float frand(void) {
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (float)((rng >> 11) % 2001) / 1000.0f - 1.0f;
}
/* n elements of dt, filled with small values (bf16: the top half of the fp32 bits) */
static void* filled(int dt, int64_t n) {
  void* p = malloc((size_t)(n > 0 ? n : 1) * (dt == BF16 ? 2 : 4));
  for (int64_t i = 0; i < n; ++i) {
    float f = frand();
    if (dt == BF16) { uint32_t u; memcpy(&u, &f, 4); ((uint16_t*)p)[i] = (uint16_t)(u >> 16); }
    else ((float*)p)[i] = f;
  }
  return p;
}
static void* out(int dt, int64_t n) { return calloc((size_t)(n > 0 ? n : 1), dt == BF16 ? 2 : 4); }

static void gemm_rs_cases(int in, int sl, int od) {
  const int P = 3, M = 6, N = 5, K = 7, Mc = M / P;
  void *A = filled(in, (int64_t)P * M * K), *W = filled(in, (int64_t)P * K * N);
  void *slots = out(sl, (int64_t)P * P * Mc * N), *o = out(od, (int64_t)M * N), *win = out(od, (int64_t)P * M * N);
  EXPECT(oracle_gemm_rs(P, M, N, K, in, sl, od, A, W, slots, o) == 0);
  EXPECT(oracle_gemm_rs(P, M, N, K, in, sl, od, A, W, NULL, o) == 0);
  EXPECT(oracle_gemm_ar(P, M, N, K, in, sl, od, A, W, slots, win) == 0);
  const int64_t ms[4] = {0, 5, 3, 1}, ns[4] = {0, 4, 2, 3};
  void *sv = out(sl, 4 * P), *ov = out(od, 4);
  EXPECT(oracle_gemm_rs_points(P, M, N, K, in, sl, od, A, W, 4, ms, ns, sv, ov) == 0);
  EXPECT(oracle_gemm_rs(P, M, 0, K, in, sl, od, A, W, slots, o) == 0);  /* no columns */
  EXPECT(oracle_gemm_rs(P, M, N, 0, in, sl, od, A, W, slots, o) == 0);  /* empty sum */
  EXPECT(oracle_gemm_rs(P, 0, N, K, in, sl, od, A, W, slots, o) == 0);  /* no rows */
  EXPECT(oracle_gemm_rs(P, 7, N, K, in, sl, od, A, W, slots, o) == -1); /* M not a multiple of P */
  EXPECT(oracle_gemm_rs(0, M, N, K, in, sl, od, A, W, slots, o) == -1);
  free(A); free(W); free(slots); free(o); free(win); free(sv); free(ov);
}

static void gemv_ag_cases(int in, int od) {
  const int P = 3, Mb = 2, N = 5, K = 7, Mc = 2;
  void *x = filled(in, (int64_t)P * Mb * K), *W = filled(in, (int64_t)P * K * N);
  void *part = out(F32, (int64_t)P * Mb * N), *win = out(od, (int64_t)P * Mb * N);
  EXPECT(oracle_gemv_ar(P, Mb, N, K, in, F32, od, x, W, part, win) == 0);
  EXPECT(oracle_gemv_ar(P, Mb, N, K, in, F32, od, x, W, NULL, win) == 0);
  EXPECT(oracle_gemv_ar(P, 0, N, K, in, F32, od, x, W, part, win) == 0);
  void* chunks[3];
  for (int c = 0; c < P; ++c) chunks[c] = filled(in, (int64_t)Mc * K);
  void *Wg = filled(in, (int64_t)K * N), *g = out(in, (int64_t)P * Mc * K), *o = out(od, (int64_t)P * Mc * N);
  EXPECT(oracle_ag_gemm(P, Mc, N, K, in, od, (const void* const*)chunks, Wg, g, o) == 0);
  EXPECT(oracle_ag_gemm(P, Mc, N, K, in, od, (const void* const*)chunks, Wg, NULL, o) == 0);
  const int64_t ms[3] = {0, 5, 2}, ns[3] = {4, 0, 2};
  void* ov = out(od, 3);
  EXPECT(oracle_ag_gemm_points(P, Mc, N, K, in, od, (const void* const*)chunks, Wg, 3, ms, ns, ov) == 0);
  EXPECT(oracle_ag_gemm(P, 0, N, K, in, od, (const void* const*)chunks, Wg, g, o) == 0);
  for (int c = 0; c < P; ++c) free(chunks[c]);
  free(x); free(W); free(part); free(win); free(Wg); free(g); free(o); free(ov);
}

static void moe_cases(void) {
  /* combine: 2 experts, rows [0,4) and [4,8), last row of each group padding */
  const int P = 2, E = 2, N = 3, K = 5;
  const int64_t T = 8, cap = 8, offs[3] = {0, 4, 8};
  const int32_t dest[8] = {0, 1, 0, -1, 1, 0, 1, -1}, slot[8] = {0, 0, 1, -1, 1, 2, 2, -1};
  void *X = filled(BF16, T * K), *W = filled(BF16, (int64_t)E * K * N), *win = out(BF16, (int64_t)P * cap * N);
  EXPECT(oracle_gemm_a2a(P, E, T, N, K, BF16, BF16, X, W, offs, dest, slot, cap, win) == 0);
  const int32_t twice[8] = {0, 1, 0, -1, 1, 0, 1, -1}, same_slot[8] = {0, 0, 0, -1, 1, 2, 2, -1};
  EXPECT(oracle_gemm_a2a(P, E, T, N, K, BF16, BF16, X, W, offs, twice, same_slot, cap, win) == -1);
  const int32_t far_slot[8] = {0, 1, 0, -1, 1, 0, 1, 9};
  const int32_t far_dest[8] = {0, 1, 0, -1, 1, 0, 1, 1};
  EXPECT(oracle_gemm_a2a(P, E, T, N, K, BF16, BF16, X, W, offs, far_dest, far_slot, cap, win) == -1);
  free(X); free(W); free(win);
  /* dispatch: 2 sources x 5 tokens, top-2 of 4 global experts, this rank holds 0 and 1 */
  const int B = 5, topk = 2, tile_m = 4;
  const int32_t experts[20] = {0, 1, 2, 3, 1, 2, 0, 3, 3, 1, 2, 0, 1, 3, 0, 2, 3, 2, 1, 0};
  void *Xs = filled(BF16, (int64_t)P * B * K), *We = filled(BF16, (int64_t)E * K * N);
  const int64_t capd = 24;
  void *recv = out(BF16, capd * K), *Y = out(F32, capd * N);
  int64_t offsets[3], send[2];
  int32_t dd[24], ss[24];
  EXPECT(oracle_a2a_gemm(P, E, 0, B, topk, N, K, BF16, F32, Xs, experts, We, tile_m, capd, recv, Y, offsets, dd, ss,
                         send) == 0);
  EXPECT(offsets[0] == 0 && offsets[2] <= capd && send[0] + send[1] > 0);
  EXPECT(oracle_a2a_gemm(P, E, 0, B, topk, N, K, BF16, F32, Xs, experts, We, tile_m, 4, recv, Y, offsets, dd, ss,
                         send) == -1); /* more rows than the receive buffer holds */
  EXPECT(oracle_a2a_gemm(P, E, 2, B, topk, N, K, BF16, F32, Xs, experts, We, tile_m, capd, recv, Y, offsets, dd, ss,
                         send) == 0);  /* the other rank's experts */
  free(Xs); free(We); free(recv); free(Y);
}

static void embbag_cases(void) {
  const int T = 2, D = 4, B = 4, L = 3, P = 2;
  const int64_t R = 10;
  float* tab = (float*)filled(F32, T * R * D);
  int32_t idx[24];
  for (int i = 0; i < 24; ++i) idx[i] = (i * 7) % (int)R;
  float* win = (float*)out(F32, (int64_t)B * T * D);
  EXPECT(oracle_embbag_a2a(T, R, D, B, L, P, tab, idx, NULL, win) == 0);
  const int64_t csr[9] = {0, 0, 5, 5, 9, 12, 12, 20, 24};  /* empty bags included */
  EXPECT(oracle_embbag_a2a(T, R, D, B, 0, P, tab, idx, csr, win) == 0);
  idx[4] = (int32_t)R;                                      /* one index out of range */
  EXPECT(oracle_embbag_a2a(T, R, D, B, L, P, tab, idx, NULL, win) == -2);
  EXPECT(oracle_embbag_a2a(T, R, D, 3, L, P, tab, idx, NULL, win) == -1); /* B not a multiple of P */
  free(tab); free(win);
}

int main(void) {
  gemm_rs_cases(F32, F32, F32);
  gemm_rs_cases(BF16, F32, BF16);
  gemm_rs_cases(BF16, BF16, F32);
  gemv_ag_cases(BF16, BF16);
  gemv_ag_cases(F32, F32);
  moe_cases();
  embbag_cases();
  printf("oracle driver: %d failures\n", fails);
  return fails ? 1 : 0;
}
