/*
 * CPU oracle for the fused computation + collective-epilogue operators.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code with the HIP library (no headers,
 * no helpers, no tables) and generates none of its own inputs: it consumes
 * the exact bytes the GPU receives.
 *
 * What it computes.  "Optimizing Distributed ML Communication with Fused
 * Computation-Collective Operations" (SC24, abstract) fuses a computation
 * with the collective that follows it: workgroups send their results on as
 * soon as they finish, while others still compute.  Fusion changes when the
 * data moves, not what is computed, so the oracle is the unfused definition
 * written out: the per-shard computation, then the textbook collective
 * (ReduceScatter, AllReduce, AllGather, All-to-All).  The operator pairs are
 * the ones those pages name: GEMM + ReduceScatter and AllGather + GEMM (the
 * mKernel news item "GPU-vezérelt kommunikációval gyorsítják az
 * AI-betanítást a kutatók", section on the five fused kernels), GEMV +
 * AllReduce and embedding + All-to-All (SC24 abstract).
 *
 * Readings taken where the pages are silent:
 *  - per-shard products are accumulated in fp64 with k ascending, then
 *    rounded to fp32 (RNE), and from fp32 to bf16 (RNE) when the partial is
 *    carried in bf16 -- the two-step rounding of an fp32 accumulator;
 *  - partials are reduced by a left fold in fp32 in rank order
 *    p = 0, 1, ..., P-1, starting from partial 0, then rounded once to the
 *    output type;
 *  - chunk r of a ReduceScatter is the contiguous row block
 *    [r*Mc, (r+1)*Mc) of the full result; it goes to destination r; the slot
 *    inside destination r is the source rank p;
 *  - embedding bags are summed in fp32 in index order starting from +0.0;
 *    an empty bag pools to zeros; bag b goes to destination b / (B/P), slot
 *    b mod (B/P);
 *  - an AllGather concatenates the chunks in rank order, whatever the order
 *    in which they arrived.
 *
 * Data types: code 0 = fp32, code 1 = bf16 carried as uint16 bit patterns.
 * Every function returns 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define DT_F32 0
#define DT_BF16 1

/* ---- element conversions (this file's own; IEEE-754 binary32 -> bfloat16) ---- */

static float from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round an fp32 value to bfloat16, nearest-even.  bfloat16 keeps the top 16
 * bits of the binary32 pattern; the dropped 16 bits decide the rounding. */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) /* NaN: keep it quiet */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u; /* carries into the exponent correctly, up to infinity */
    return (uint16_t)upper;
}

static double load_in(const void* base, int dt, int64_t i) {
    if (dt == DT_BF16) return (double)from_bf16(((const uint16_t*)base)[i]);
    return (double)((const float*)base)[i];
}

/* Store a value that is already an fp32 number into a buffer of type dt. */
static void store_f32_as(void* base, int dt, int64_t i, float v) {
    if (dt == DT_BF16) ((uint16_t*)base)[i] = to_bf16(v);
    else ((float*)base)[i] = v;
}

/* The partial C_p[m][n] as it is carried: fp64 sum -> fp32 -> (bf16). */
static float carried(double s, int slot_dt) {
    float f = (float)s; /* RNE */
    if (slot_dt == DT_BF16) f = from_bf16(to_bf16(f));
    return f;
}

static int dt_ok(int dt) { return dt == DT_F32 || dt == DT_BF16; }

/* ---- GEMM + ReduceScatter ------------------------------------------------
 * A [P][M][K], W [P][K][N] (row-major).  Shard p computes C_p = A_p . W_p
 * (M x N).  The ReduceScatter hands chunk r (rows r*Mc .. r*Mc+Mc-1) of every
 * C_p to destination r, which folds the P partials in rank order.
 *   slots: [P dst r][P src p][Mc][N] of slot_dt (may be NULL): C_p chunk r
 *   out:   [M][N] of out_dt == [P][Mc][N]: the reduced chunks in dest order
 */
int oracle_gemm_rs(int P, int M, int N, int K, int in_dt, int slot_dt, int out_dt,
                   const void* A, const void* W, void* slots, void* out) {
    if (P <= 0 || M < 0 || N < 0 || K < 0 || M % P != 0) return -1;
    if (!dt_ok(in_dt) || !dt_ok(slot_dt) || !dt_ok(out_dt)) return -1;
    const int64_t Mc = M / P;
    /* carried partials C_p, fp32 values after the slot rounding: [P][M][N] */
    float* C = (float*)malloc(sizeof(float) * (size_t)P * (size_t)M * (size_t)(N > 0 ? N : 1));
    if (!C) return -1;

    /* 1. per-shard GEMM, fp64, k ascending */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pm = 0; pm < (int64_t)P * M; ++pm) {
        const int64_t p = pm / M, m = pm % M;
        double* acc = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_in(A, in_dt, (p * M + m) * K + k);
            const int64_t wrow = (p * K + k) * N;
            for (int64_t n = 0; n < N; ++n) acc[n] += a * load_in(W, in_dt, wrow + n);
        }
        for (int64_t n = 0; n < N; ++n) C[(p * M + m) * N + n] = carried(acc[n], slot_dt);
        free(acc);
    }

    /* 2. scatter: chunk r of C_p -> destination r, slot p */
    if (slots) {
        for (int64_t r = 0; r < P; ++r)
            for (int64_t p = 0; p < P; ++p)
                for (int64_t i = 0; i < Mc; ++i)
                    for (int64_t n = 0; n < N; ++n)
                        store_f32_as(slots, slot_dt, ((r * P + p) * Mc + i) * N + n,
                                     C[(p * M + r * Mc + i) * N + n]);
    }

    /* 3. each destination folds its P slots in rank order, in fp32 */
    for (int64_t r = 0; r < P; ++r)
        for (int64_t i = 0; i < Mc; ++i)
            for (int64_t n = 0; n < N; ++n) {
                const int64_t m = r * Mc + i;
                float acc = C[(0 * M + m) * N + n];
                for (int64_t p = 1; p < P; ++p) acc = acc + C[(p * M + m) * N + n];
                store_f32_as(out, out_dt, m * N + n, acc);
            }
    free(C);
    return 0;
}

/* Sampled GEMM + ReduceScatter: the same definition evaluated at npts output
 * coordinates (m[i], n[i]) only.  slot_vals: [npts][P] of slot_dt (may be
 * NULL) = C_p[m][n] as carried; out_vals: [npts] of out_dt. */
int oracle_gemm_rs_points(int P, int M, int N, int K, int in_dt, int slot_dt, int out_dt,
                          const void* A, const void* W, int64_t npts, const int64_t* ms,
                          const int64_t* ns, void* slot_vals, void* out_vals) {
    if (P <= 0 || M % P != 0 || !dt_ok(in_dt) || !dt_ok(slot_dt) || !dt_ok(out_dt)) return -1;
    for (int64_t i = 0; i < npts; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t m = ms[i], n = ns[i];
        float acc = 0.0f;
        for (int64_t p = 0; p < P; ++p) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += load_in(A, in_dt, (p * M + m) * K + k) * load_in(W, in_dt, (p * K + k) * N + n);
            const float c = carried(s, slot_dt);
            if (slot_vals) store_f32_as(slot_vals, slot_dt, i * P + p, c);
            acc = (p == 0) ? c : acc + c;
        }
        store_f32_as(out_vals, out_dt, i, acc);
    }
    return 0;
}

/* ---- GEMM + AllReduce -----------------------------------------------------
 * The mKernel news item lists GEMM + AllReduce among its five fused kernels
 * (section on the fused kernels).  A [P][M][K], W [P][K][N].  Shard p
 * computes C_p = A_p . W_p (M x N), carried in slot_dt.  The AllReduce
 * leaves the sum of the P partials -- folded in rank order in fp32, rounded
 * once to out_dt -- in every one of the P receive windows.  It is carried out
 * in two phases: a ReduceScatter (chunk r of every C_p to destination r,
 * slot p, folded there) and an AllGather of the reduced chunks, so every
 * window ends up holding all M rows with the same bits.
 *   slots: [P dst r][P src p][Mc][N] of slot_dt (may be NULL): C_p chunk r
 *   win:   [P dst q][M][N] of out_dt: the full reduced result, once per q
 */
int oracle_gemm_ar(int P, int M, int N, int K, int in_dt, int slot_dt, int out_dt,
                   const void* A, const void* W, void* slots, void* win) {
    if (P <= 0 || M < 0 || N < 0 || K < 0 || M % P != 0) return -1;
    if (!dt_ok(in_dt) || !dt_ok(slot_dt) || !dt_ok(out_dt)) return -1;
    const int64_t Mc = M / P;
    float* C = (float*)malloc(sizeof(float) * (size_t)P * (size_t)M * (size_t)(N > 0 ? N : 1));
    if (!C) return -1;

    /* 1. per-shard GEMM, fp64, k ascending, carried in slot_dt */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pm = 0; pm < (int64_t)P * M; ++pm) {
        const int64_t p = pm / M, m = pm % M;
        double* acc = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_in(A, in_dt, (p * M + m) * K + k);
            const int64_t wrow = (p * K + k) * N;
            for (int64_t n = 0; n < N; ++n) acc[n] += a * load_in(W, in_dt, wrow + n);
        }
        for (int64_t n = 0; n < N; ++n) C[(p * M + m) * N + n] = carried(acc[n], slot_dt);
        free(acc);
    }

    /* 2. ReduceScatter phase: chunk r of C_p -> destination r, slot p */
    if (slots) {
        for (int64_t r = 0; r < P; ++r)
            for (int64_t p = 0; p < P; ++p)
                for (int64_t i = 0; i < Mc; ++i)
                    for (int64_t n = 0; n < N; ++n)
                        store_f32_as(slots, slot_dt, ((r * P + p) * Mc + i) * N + n,
                                     C[(p * M + r * Mc + i) * N + n]);
    }

    /* 3. destination r folds its chunk in rank order; 4. AllGather phase:
     * the reduced chunk r lands at rows r*Mc.. of every window q */
    for (int64_t r = 0; r < P; ++r)
        for (int64_t i = 0; i < Mc; ++i)
            for (int64_t n = 0; n < N; ++n) {
                const int64_t m = r * Mc + i;
                float acc = C[(0 * M + m) * N + n];
                for (int64_t p = 1; p < P; ++p) acc = acc + C[(p * M + m) * N + n];
                for (int64_t q = 0; q < P; ++q) store_f32_as(win, out_dt, (q * M + m) * N + n, acc);
            }
    free(C);
    return 0;
}

/* ---- GEMM + All-to-All ----------------------------------------------------
 * SC24 (abstract) names GEMM + All-to-All, for mixture-of-experts layers,
 * among its three fused prototypes.  This rank holds E experts and has
 * received, for each expert e, a group of token rows X[offsets[e] ..
 * offsets[e+1]) (rows of expert e, [K] each).  Each row is multiplied by its
 * expert's W_e [K][N] (fp64, k ascending, rounded once to out_dt), and the
 * All-to-All sends the result row back to the token's rank: row i lands in
 * window dest[i] at slot slot[i].  A row with dest[i] < 0 is padding and
 * goes nowhere.
 *   X [T][K], W [E][K][N] of in_dt; offsets [E+1] int64 non-decreasing from
 *   0 to T; dest, slot [T] int32; win [P][cap][N] of out_dt.
 * Every (dest, slot) pair may be written at most once: a repeated pair, a
 * dest >= P or a slot outside [0, cap) is an error (-1). */
int oracle_gemm_a2a(int P, int E, int64_t T, int N, int K, int in_dt, int out_dt, const void* X,
                    const void* W, const int64_t* offsets, const int32_t* dest, const int32_t* slot,
                    int64_t cap, void* win) {
    if (P <= 0 || E <= 0 || T < 0 || N < 0 || K < 0 || cap < 0) return -1;
    if (!dt_ok(in_dt) || !dt_ok(out_dt)) return -1;
    if (offsets[0] != 0 || offsets[E] != T) return -1;
    for (int e = 0; e < E; ++e)
        if (offsets[e + 1] < offsets[e]) return -1;
    /* routing: each real row names one (dest, slot), and no pair is named twice */
    unsigned char* used = (unsigned char*)calloc((size_t)(P * cap > 0 ? P * cap : 1), 1);
    if (!used) return -1;
    for (int64_t i = 0; i < T; ++i) {
        if (dest[i] < 0) continue;
        if (dest[i] >= P || slot[i] < 0 || slot[i] >= cap || used[dest[i] * cap + slot[i]]) {
            free(used);
            return -1;
        }
        used[dest[i] * cap + slot[i]] = 1;
    }
    free(used);

    /* expert GEMM per row, then the row goes to its (dest, slot) */
    for (int e = 0; e < E; ++e) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = offsets[e]; i < offsets[e + 1]; ++i) {
            if (dest[i] < 0) continue;
            double* acc = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
            for (int64_t k = 0; k < K; ++k) {
                const double a = load_in(X, in_dt, i * K + k);
                const int64_t wrow = ((int64_t)e * K + k) * N;
                for (int64_t n = 0; n < N; ++n) acc[n] += a * load_in(W, in_dt, wrow + n);
            }
            const int64_t base = ((int64_t)dest[i] * cap + slot[i]) * N;
            for (int64_t n = 0; n < N; ++n) store_f32_as(win, out_dt, base + n, (float)acc[n]);
            free(acc);
        }
    }
    return 0;
}

/* ---- All-to-All + GEMM (MoE dispatch + GEMM) -------------------------------
 * The mKernel news item (section on its five fused kernels) lists MoE
 * Dispatch + GEMM: the All-to-All that delivers each token row to the rank
 * holding each expert its router picked, followed by the expert GEMM.  One
 * rank's share: P source ranks each hold B tokens X[p][b] ([K] each) and
 * their top-k choices experts[p][b][j] (global expert ids); this rank owns
 * experts e0 .. e0+E-1.
 * Dispatch (this rank's side of the All-to-All, the standard semantics: what
 * every source sends here, in source-rank order):
 *   - the rows of local expert e are the pairs (p, b, j) with
 *     experts[p][b][j] == e0 + e, in (p, b, j) order;
 *   - the groups follow one another in expert order, each padded with zero
 *     rows to a multiple of tile_m (the block-aligned layout of a grouped
 *     GEMM): offsets[0] = 0, offsets[e+1] = offsets[e] + ceil(n_e / tile_m)
 *     * tile_m;
 *   - recv[offsets[e] + i] = X[p][b] for the i-th pair of expert e;
 *   - dest[row] = p (where the result goes back) and slot[row] = the pair's
 *     position among source p's pairs that land here, in (b, j) order;
 *     padding rows have dest = slot = -1; send_counts[p] = source p's pairs
 *     that land here.
 * GEMM: Y[row] = recv[row] . W_e (fp64, k ascending, rounded once to out_dt),
 * padding rows included (they are zero).
 *   X [P][B][K], W [E][K][N] of in_dt; experts [P][B][topk] int32 (ids outside
 *   [e0, e0+E) are other ranks' experts); recv [cap][K] of in_dt, Y [cap][N]
 *   of out_dt, dest and slot [cap] int32, offsets [E+1] and send_counts [P]
 *   int64.  Rows from offsets[E] to cap are left as they were;
 *   offsets[E] > cap is an error (-1, nothing written). */
int oracle_a2a_gemm(int P, int E, int e0, int B, int topk, int N, int K, int in_dt, int out_dt,
                    const void* X, const int32_t* experts, const void* W, int tile_m, int64_t cap,
                    void* recv, void* Y, int64_t* offsets, int32_t* dest, int32_t* slot,
                    int64_t* send_counts) {
    if (P <= 0 || E <= 0 || B < 0 || topk < 0 || N < 0 || K < 0 || tile_m <= 0 || cap < 0) return -1;
    if (!dt_ok(in_dt) || !dt_ok(out_dt)) return -1;
    const int in_es = in_dt == DT_BF16 ? 2 : 4;

    /* pairs per local expert, then the padded group offsets */
    int64_t* n = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* next = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    if (!n || !next) { free(n); free(next); return -1; }
    for (int64_t i = 0; i < (int64_t)P * B * topk; ++i) {
        const int64_t e = (int64_t)experts[i] - e0;
        if (e >= 0 && e < E) n[e] += 1;
    }
    int64_t total = 0;
    for (int e = 0; e < E; ++e) total += (n[e] + tile_m - 1) / tile_m * tile_m;
    if (total > cap) { free(n); free(next); return -1; }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + (n[e] + tile_m - 1) / tile_m * tile_m;

    /* every pair in (p, b, j) order takes the next row of its expert's group */
    for (int p = 0; p < P; ++p) {
        int64_t s = 0;   /* source p's pairs that land here so far */
        for (int b = 0; b < B; ++b)
            for (int j = 0; j < topk; ++j) {
                const int64_t e = (int64_t)experts[((int64_t)p * B + b) * topk + j] - e0;
                if (e < 0 || e >= E) continue;
                const int64_t row = offsets[e] + next[e]++;
                memcpy((char*)recv + row * K * in_es, (const char*)X + ((int64_t)p * B + b) * K * in_es,
                       (size_t)K * in_es);
                dest[row] = p;
                slot[row] = (int32_t)s++;
            }
        send_counts[p] = s;
    }
    /* the padding rows of every group */
    for (int e = 0; e < E; ++e)
        for (int64_t row = offsets[e] + n[e]; row < offsets[e + 1]; ++row) {
            memset((char*)recv + row * K * in_es, 0, (size_t)K * in_es);
            dest[row] = -1;
            slot[row] = -1;
        }
    free(n);
    free(next);

    /* the expert GEMM, row by row */
    for (int e = 0; e < E; ++e) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t row = offsets[e]; row < offsets[e + 1]; ++row) {
            double* acc = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
            for (int64_t k = 0; k < K; ++k) {
                const double a = load_in(recv, in_dt, row * K + k);
                const int64_t wrow = ((int64_t)e * K + k) * N;
                for (int64_t c = 0; c < N; ++c) acc[c] += a * load_in(W, in_dt, wrow + c);
            }
            for (int64_t c = 0; c < N; ++c) store_f32_as(Y, out_dt, row * N + c, (float)acc[c]);
            free(acc);
        }
    }
    return 0;
}

/* ---- GEMV + AllReduce -----------------------------------------------------
 * x [P][Mb][K], W [P][K][N].  Shard p computes y_p = x_p . W_p (Mb x N),
 * carried in slot_dt; the AllReduce folds y_0..y_{P-1} in rank order in fp32,
 * rounds once to out_dt and leaves the same result in every one of the P
 * receive windows.
 *   part: [P][Mb][N] of slot_dt (may be NULL); win: [P][Mb][N] of out_dt */
int oracle_gemv_ar(int P, int Mb, int N, int K, int in_dt, int slot_dt, int out_dt,
                   const void* x, const void* W, void* part, void* win) {
    if (P <= 0 || Mb < 0 || N < 0 || K < 0) return -1;
    if (!dt_ok(in_dt) || !dt_ok(slot_dt) || !dt_ok(out_dt)) return -1;
    float* Y = (float*)malloc(sizeof(float) * (size_t)P * (size_t)(Mb > 0 ? Mb : 1) * (size_t)(N > 0 ? N : 1));
    if (!Y) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pb = 0; pb < (int64_t)P * Mb; ++pb) {
        const int64_t p = pb / Mb, b = pb % Mb;
        double* acc = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_in(x, in_dt, (p * Mb + b) * K + k);
            const int64_t wrow = (p * K + k) * N;
            for (int64_t n = 0; n < N; ++n) acc[n] += a * load_in(W, in_dt, wrow + n);
        }
        for (int64_t n = 0; n < N; ++n) Y[(p * Mb + b) * N + n] = carried(acc[n], slot_dt);
        free(acc);
    }
    if (part)
        for (int64_t i = 0; i < (int64_t)P * Mb * N; ++i) store_f32_as(part, slot_dt, i, Y[i]);
    for (int64_t b = 0; b < Mb; ++b)
        for (int64_t n = 0; n < N; ++n) {
            float acc = Y[(0 * Mb + b) * N + n];
            for (int64_t p = 1; p < P; ++p) acc = acc + Y[(p * Mb + b) * N + n];
            for (int64_t q = 0; q < P; ++q) store_f32_as(win, out_dt, (q * Mb + b) * N + n, acc);
        }
    free(Y);
    return 0;
}

/* ---- AllGather + GEMM -----------------------------------------------------
 * chunks: P pointers, chunk c = [Mc][K] held by rank c; W [K][N].
 * The AllGather builds A_g = [chunk 0; chunk 1; ...; chunk P-1] (rank order);
 * then out = A_g . W, fp64 accumulation, rounded to fp32 then to out_dt.
 *   gathered: [P*Mc][K] of in_dt (may be NULL); out: [P*Mc][N] of out_dt */
int oracle_ag_gemm(int P, int Mc, int N, int K, int in_dt, int out_dt,
                   const void* const* chunks, const void* W, void* gathered, void* out) {
    if (P <= 0 || Mc < 0 || N < 0 || K < 0 || !dt_ok(in_dt) || !dt_ok(out_dt)) return -1;
    const size_t esz = in_dt == DT_BF16 ? 2 : 4;
    const int64_t M = (int64_t)P * Mc;
    char* Ag = (char*)malloc(esz * (size_t)(M > 0 ? M : 1) * (size_t)(K > 0 ? K : 1));
    if (!Ag) return -1;
    for (int64_t c = 0; c < P; ++c) /* rank order */
        memcpy(Ag + (size_t)c * Mc * K * esz, chunks[c], (size_t)Mc * K * esz);
    if (gathered) memcpy(gathered, Ag, (size_t)M * K * esz);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        double* acc = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_in(Ag, in_dt, m * K + k);
            for (int64_t n = 0; n < N; ++n) acc[n] += a * load_in(W, in_dt, k * N + n);
        }
        for (int64_t n = 0; n < N; ++n) store_f32_as(out, out_dt, m * N + n, (float)acc[n]);
        free(acc);
    }
    free(Ag);
    return 0;
}

/* Sampled AllGather + GEMM at output coordinates (ms[i], ns[i]). */
int oracle_ag_gemm_points(int P, int Mc, int N, int K, int in_dt, int out_dt,
                          const void* const* chunks, const void* W, int64_t npts,
                          const int64_t* ms, const int64_t* ns, void* out_vals) {
    if (P <= 0 || Mc <= 0 || !dt_ok(in_dt) || !dt_ok(out_dt)) return -1;
    for (int64_t i = 0; i < npts; ++i)
        if (ms[i] < 0 || ms[i] >= (int64_t)P * Mc || ns[i] < 0 || ns[i] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t c = ms[i] / Mc, row = ms[i] % Mc, n = ns[i];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += load_in(chunks[c], in_dt, row * K + k) * load_in(W, in_dt, k * N + n);
        store_f32_as(out_vals, out_dt, i, (float)s);
    }
    return 0;
}

/* ---- embedding bag + All-to-All ------------------------------------------
 * tables [T][R][D] fp32; indices: fixed-length bags [T][B][L] (offsets NULL)
 * or CSR bags (offsets [T*B+1], bag (t,b) = indices[offsets[t*B+b] ..
 * offsets[t*B+b+1]) ).  pooled(t,b) = sum of the bag's rows, fp32, in index
 * order from +0.0.  The All-to-All sends bag b to destination d = b / Bd
 * (Bd = B/P), slot b mod Bd:
 *   win: [P][Bd][T][D] fp32, win[d][b mod Bd][t][:] = pooled(t, b).
 * An index outside [0, R) makes the call fail (-2) and leaves win unspecified. */
int oracle_embbag_a2a(int T, int64_t R, int D, int B, int L, int P, const float* tables,
                      const int32_t* indices, const int64_t* offsets, float* win) {
    if (T < 0 || R < 0 || D < 0 || B < 0 || P <= 0 || B % P != 0) return -1;
    if (!offsets && L < 0) return -1;
    const int64_t Bd = B / P;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t tb = 0; tb < (int64_t)T * B; ++tb) {
        const int64_t t = tb / B, b = tb % B;
        const int64_t lo = offsets ? offsets[tb] : tb * (int64_t)L;
        const int64_t hi = offsets ? offsets[tb + 1] : lo + L;
        float* dst = win + (((b / Bd) * Bd + (b % Bd)) * T + t) * (int64_t)D;
        for (int64_t d = 0; d < D; ++d) dst[d] = 0.0f;
        for (int64_t j = lo; j < hi; ++j) {
            const int64_t row = indices[j];
            if (row < 0 || row >= R) { bad = 1; continue; }
            const float* src = tables + (t * R + row) * (int64_t)D;
            for (int64_t d = 0; d < D; ++d) dst[d] = dst[d] + src[d];
        }
    }
    return bad ? -2 : 0;
}

/* Thread control for the timing harness (no arithmetic): the OpenMP runtime
   may already be initialised by the host process, so the environment
   variable alone does not reach it. */
void oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}
int oracle_max_threads(void) { return omp_get_max_threads(); }
