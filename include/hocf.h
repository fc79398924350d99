/*
 * hocf — computations fused with their collective epilogue, on one MI355X.
 *
 * C ABI of libhocf.so.  Seven operators, each one GPU's share of a P-way
 * tensor-parallel (or model-parallel) step with the P logical shards'
 * receive windows in local HBM, their baselines, and a put that moves such
 * traffic on the copy engines:
 *
 *   hocf_gemm_rs     GEMM + ReduceScatter   (mKernel news item "GPU-vezérelt
 *                    kommunikációval gyorsítják az AI-betanítást a kutatók",
 *                    section on its five fused kernels)
 *   hocf_gemm_ar     GEMM + AllReduce       (mKernel news item, same section)
 *   hocf_gemm_rs_unfused, hocf_gemv_ar_unfused, hocf_a2a_gemm_unfused
 *                    the same operators as separate kernels, the computation
 *                    and the collective one after the other (the baseline
 *                    SC24 measures its fused operators against)
 *   hocf_gemm_rs_noalloc
 *                    GEMM + ReduceScatter for callers that cannot allocate
 *   hocf_gemm_rs_decomposed
 *                    the same GEMM + ReduceScatter in column pieces pipelined
 *                    on two streams (Compass, abstract: InterDecom)
 *   hocf_gemv_ar     GEMV + AllReduce       ("Optimizing Distributed ML
 *                    Communication with Fused Computation-Collective
 *                    Operations", SC24, abstract)
 *   hocf_ag_gemm     AllGather + GEMM       (mKernel news item, same section)
 *   hocf_embbag_a2a  embedding bag + All-to-All (SC24 abstract)
 *   hocf_gemm_a2a    GEMM + All-to-All, the MoE combine (SC24 abstract)
 *   hocf_a2a_gemm    All-to-All + GEMM, the MoE dispatch (mKernel news item,
 *                    section on its five fused kernels)
 *   hocf_dma_put     point-to-point puts (optionally signalled) moved by
 *                    the copy (SDMA) engines instead of the compute units
 *                    ("HOCCL: Offloading Collective Communication from GPU
 *                    Cores to Accelerate Distributed Training", abstract)
 *
 * The method (SC24 abstract; mKernel, section on persistent kernels and
 * tile/chunk overlap): the workgroups of one kernel each finish an output
 * tile and immediately publish it to its destination's receive window with
 * a per-tile ready flag, while other workgroups of the same kernel are still
 * computing; the collective's consumer side (a fixed rank-order reduction,
 * or a gather-gated GEMM) consumes tiles as their flags arrive.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor, window, flag array, workspace and status pointer
 * is a device pointer on the current HIP device, 16-byte aligned, except
 * sync->abort_flag (device or host-pinned memory) and the hocf_window arrays
 * themselves (host memory, read during the call).  All tensors are dense
 * row-major.  bf16 tensors hold bfloat16 bit patterns (uint16).
 *
 * Streams.  A call validates its arguments, enqueues its kernel (the
 * unfused baselines: its two kernels) on `stream`
 * (a hipStream_t; NULL = the null stream) and returns.  Results, windows and
 * flags are valid once the stream has reached the kernel's end.  The library
 * never allocates, frees or synchronises in a call, and keeps no pointer
 * after the kernel ends.  The caller owns every buffer.
 *
 * Synchronous errors.  An invalid shape, an unsupported combination, a NULL
 * or misaligned pointer, a zero epoch, a short workspace, or aliasing
 * returns an error code BEFORE anything is enqueued; hocf_last_error() then
 * describes it.  Aliasing: every byte range a call writes (outputs, windows
 * and their flags, partials, the workspace, the status word) may overlap no
 * other range of the same call, read or written (HOCF_ERR_INVALID_ARG);
 * ranges that are only read may overlap each other.  A launch failure
 * returns HOCF_ERR_HIP.
 *
 * Asynchronous errors.  A wait that exceeds its time limit, an abort request
 * or an out-of-range embedding index is recorded in *sync->status (if
 * non-NULL) by the first workgroup that meets it (compare-and-swap from 0);
 * every workgroup still exits, and the outputs are then unspecified.  The
 * caller zeroes *status before the call and reads it after.  Every wait of
 * every operator (a flag or ready word that has not arrived yet) polls the
 * abort word too and ends with HOCF_ERR_ABORTED once it is nonzero; a call
 * that happens not to wait completes normally whatever the abort word
 * holds.
 *
 * Flags.  Flag words are uint32 and hold an epoch: a word equals
 * sync->epoch once the data it guards is complete and visible device-wide.
 * The library's producers write guarded data with device-coherent stores
 * and wait for their completion before the flag store; a consumer that sees
 * the epoch (agent-scope atomic load) and then reads the data either with
 * device-coherent loads or after an agent-scope acquire fence sees it all.
 * Each call must use an epoch different from the previous call on the same
 * flag arrays, so flags never need resetting.
 *
 * Grid.  Each call launches one persistent kernel with as many workgroups
 * as the device holds at once, capped by the number of work items.  The
 * environment variable HOCF_MAX_WORKGROUPS (a positive integer, read at each
 * call) caps it further, e.g. to leave CUs to other work or to have each
 * workgroup take many items; every operator completes with any grid of one
 * or more workgroups.
 *
 * Workspace.  Scheduler counters.  The caller allocates at least the size
 * the matching *_workspace_bytes() query returns, zeroes it ONCE, and may
 * then reuse it for any number of calls: every call leaves it zeroed again.
 * Calls that may run concurrently need separate workspaces.
 */
#ifndef HOCF_H
#define HOCF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HOCF_ABI_VERSION 1
#define HOCF_MAX_P 16 /* largest shard count any operator accepts */

/* In C++ the enums below take int as their fixed underlying type, so that
 * every int a C caller passes is a value of the type (the library checks
 * it; an enum without a fixed type would leave out-of-range values
 * undefined in C++).  The ABI is int either way. */
#ifdef __cplusplus
#define HOCF_ENUM_INT : int
#else
#define HOCF_ENUM_INT
#endif

typedef enum hocf_status HOCF_ENUM_INT {
    HOCF_OK = 0,
    HOCF_ERR_INVALID_ARG = 1, /* bad shape, pointer, alignment, epoch or workspace */
    HOCF_ERR_UNSUPPORTED = 2, /* valid, but no kernel for this combination */
    HOCF_ERR_HIP = 3,         /* a HIP runtime call failed (launch, attribute query) */
    HOCF_ERR_TIMEOUT = 4,     /* (async) a flag wait exceeded sync->spin_timeout_ns */
    HOCF_ERR_ABORTED = 5,     /* (async) *sync->abort_flag became nonzero during a wait */
    HOCF_ERR_BAD_INDEX = 6,   /* (async) an embedding index outside [0, R) was skipped */
    HOCF_ERR_PROTOCOL = 7,    /* (async) a reducer found a partial's flag not set */
    HOCF_ERR_CAPACITY = 8     /* (async) more rows routed here than the receive buffer holds */
} hocf_status;

typedef enum hocf_dtype HOCF_ENUM_INT { HOCF_F32 = 0, HOCF_BF16 = 1 } hocf_dtype;

/* One destination's receive window: its data buffer and its flag words. */
typedef struct hocf_window {
    void* data;
    uint32_t* flags;
} hocf_window;

typedef struct hocf_sync {
    uint32_t epoch;               /* nonzero; differs from the previous call on the same flags */
    uint32_t* status;             /* nullable device word; first asynchronous error code */
    const uint32_t* abort_flag;   /* nullable device or host-pinned word; nonzero ends every wait */
    uint64_t spin_timeout_ns;     /* bound of every flag wait; 0 = 1 second */
    void* workspace;              /* scheduler counters, zeroed once by the caller */
    size_t workspace_bytes;
} hocf_sync;

/* ------------------------------------------------------------------------
 * GEMM + ReduceScatter.
 *
 * Computes, for every logical shard p < P, the partial C_p = A_p . W_p
 * (M x N, fp32 accumulation) and reduce-scatters it: chunk r (rows
 * [r*Mc, (r+1)*Mc), Mc = M/P) of every C_p goes to destination r, slot p,
 * and destination r folds its P slots in rank order p = 0..P-1 in fp32,
 * rounding once to out_dt.  Each workgroup that finishes a tile of C_p
 * publishes it into win[r] (slot_dt) and sets its flag; once all P
 * producers of an output tile have published, the tile's fold (in bands of
 * rows) is taken up by workgroups of the same kernel, mostly during their
 * next tile's mainloop, while other workgroups still compute.
 *
 *   A    [P][M][K] in_dt          W  [P][K][N] in_dt
 *   win  host array of P windows; win[r].data = [P src][Mc][N] slot_dt,
 *        win[r].flags = [P src][Tc] with Tc = ceil(Mc/tile_m) * ceil(N/tile_n);
 *        flag (p, t) = epoch once tile t (row-major over the chunk's tile
 *        grid) of C_p's chunk r is in slot p of window r
 *   out  [M][N] out_dt  (= [P][Mc][N]: destination r's reduced chunk at rows r*Mc)
 *
 * Supported: (in, slot, out) = (F32, F32, F32) with tile 64x64;
 *            (BF16, F32 or BF16, BF16 or F32) with tiles 256x256 and 128x128.
 * Requires M % P == 0; N and K multiples of 8 (bf16) or 4 (fp32).  Tiles may
 * be ragged at the end of a chunk, of N and of K.  M, N or K may be 0.
 * HOCF_ERR_UNSUPPORTED when tile_m * N reaches 2^29 elements (a tile's row
 * band is addressed with 32-bit byte offsets).
 * ---------------------------------------------------------------------- */
hocf_status hocf_gemm_rs(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                         hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                         void* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream);
size_t hocf_gemm_rs_workspace_bytes(int P, int M, int N, int tile_m, int tile_n);

/* ------------------------------------------------------------------------
 * GEMM + ReduceScatter that allocates nothing.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * operator, arguments, arithmetic and results as hocf_gemm_rs (bit for bit),
 * except that the scheduler words the workspace holds come from a scratch
 * array of HOCF_NOALLOC_SCRATCH_BYTES inside the library, one per device,
 * held until the process ends.  sync->workspace must be NULL and
 * sync->workspace_bytes 0; the caller still passes every input, output,
 * window and flag array.  Each call first zeroes the scratch words it uses
 * (with a kernel on `stream`, no memset), then enqueues the operator's
 * kernel; neither the call nor the library ever calls hipMalloc or hipFree.
 *
 * The scratch is shared by every call on a device: calls that may overlap
 * on one device (different streams, or graphs replayed concurrently) race
 * and give unspecified results.  A shape whose scheduler words
 * (hocf_gemm_rs_workspace_bytes) exceed the scratch returns
 * HOCF_ERR_UNSUPPORTED before anything is enqueued: the limit is some 29,000
 * output tiles x shards, e.g. the 8-shard 8192 x 4096 workload with 256 x 256
 * tiles needs 147 KB.  Other errors as for hocf_gemm_rs.
 * ---------------------------------------------------------------------- */
#define HOCF_NOALLOC_SCRATCH_BYTES (1u << 20)
hocf_status hocf_gemm_rs_noalloc(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                                 hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                                 void* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream);

/* ------------------------------------------------------------------------
 * GEMM + ReduceScatter, unfused (the baseline the fused operator is
 * measured against).
 *
 * SC24 (abstract) reports its fused operators against running the
 * computation and then the collective; the mKernel item contrasts its
 * in-kernel tile overlap with the same.  This entry point is that
 * bulk-synchronous form on one GPU: the same arguments, arithmetic and
 * results as hocf_gemm_rs (bit for bit: the same per-tile products and the
 * same rank-order fold), computed by two kernels enqueued back to back on
 * `stream` -- the GEMM, which publishes every tile of every C_p into its
 * slot of win[r] and does nothing else, and then a fold kernel that reduces
 * every destination's P slots in rank order into `out` once the GEMM kernel
 * has ended.  No tile flag is written (win[r].flags is left as it was) and
 * no fold overlaps the GEMM.  Supported combinations, limits, workspace
 * (hocf_gemm_rs_workspace_bytes) and errors as for hocf_gemm_rs.
 * ---------------------------------------------------------------------- */
hocf_status hocf_gemm_rs_unfused(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                                 hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                                 void* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream);

/* ------------------------------------------------------------------------
 * GEMM + ReduceScatter, decomposed (the inter-operator decomposition of
 * "Compass: Dissecting Communication and Computation Operators for
 * Efficient LLM Training", abstract: the tensor split into parts whose
 * computation and communication are pipelined, the number of parts being
 * the decomposition degree).
 *
 * The same arguments, arithmetic and results as hocf_gemm_rs, bit for bit
 * (the same tile products and the same rank-order fold), computed as
 * `pieces` column pieces: piece i is columns [i*N/pieces, (i+1)*N/pieces)
 * of every partial and of the output.  Its shard GEMMs (the unfused GEMM
 * kernel, publishing into the piece's columns of the slots) run on `stream`
 * with the grid capped to leave `fold_cus` compute units free (0: no cap);
 * its fold runs on `coll_stream` once that GEMM kernel has ended (an event),
 * while piece i+1's GEMMs run on `stream`.  `stream` then waits for the
 * last fold, so the results are complete when `stream` reaches the end of
 * the call.  No tile flag is written.  `coll_stream` may equal `stream`
 * (then nothing overlaps).  The library keeps 17 HIP events per device,
 * created at its first call and reused by every later one.
 *
 * Requires 1 <= pieces <= 16 and N a multiple of pieces * tile_n
 * (else HOCF_ERR_UNSUPPORTED); supported combinations, limits, workspace
 * (hocf_gemm_rs_workspace_bytes) and errors as for hocf_gemm_rs.
 * ---------------------------------------------------------------------- */
hocf_status hocf_gemm_rs_decomposed(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                                    hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                                    void* out, int tile_m, int tile_n, int pieces, int fold_cus,
                                    const hocf_sync* sync, void* stream, void* coll_stream);

/* ------------------------------------------------------------------------
 * GEMM + AllReduce.
 *
 * The mKernel news item ("GPU-vezérelt kommunikációval gyorsítják az
 * AI-betanítást a kutatók", section on the five fused kernels) lists GEMM +
 * AllReduce among its fused kernels.  Same computation and ReduceScatter
 * phase as hocf_gemm_rs -- C_p = A_p . W_p for every shard p, chunk r of
 * every C_p published into win[r], slot p, with its tile flags, and folded
 * there in rank order p = 0..P-1 in fp32 by workgroups of the same kernel
 * while others still compute -- and then each folded band is stored into
 * every one of the P output windows (the AllGather phase), so every
 * destination holds the whole sum, the same bits in all P.
 *
 *   A, W, win      as for hocf_gemm_rs
 *   out            host array of P device pointers; out[q] = [M][N] out_dt,
 *                  destination q's copy of the full result (rows r*Mc.. are
 *                  the fold of chunk r); the P ranges must not overlap
 *
 * Supported combinations, limits and errors as for hocf_gemm_rs; the
 * workspace is the same size (hocf_gemm_ar_workspace_bytes).  The outputs
 * carry no flags: they are complete when the stream reaches the end of the
 * call.  The library keeps no pointer from `out` after the call returns (the
 * P pointers are copied into the launch's arguments).
 * ---------------------------------------------------------------------- */
hocf_status hocf_gemm_ar(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                         hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                         void* const* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream);
size_t hocf_gemm_ar_workspace_bytes(int P, int M, int N, int tile_m, int tile_n);

/* ------------------------------------------------------------------------
 * GEMV + AllReduce.
 *
 * y_p = x_p . W_p (Mb x N, fp32 accumulation) for every shard p; the
 * AllReduce folds y_0..y_{P-1} in rank order in fp32, rounds once to out_dt
 * and writes the same bits into every one of the P receive windows.
 *
 *   x     [P][Mb][K] in_dt        W  [P][K][N] in_dt
 *   part  [P][Mb][N] slot_dt: the published partials
 *   part_flags [P][NT], NT = ceil(N/tile_n): epoch once partial tile (p, j) is in part
 *   win   host array of P windows; win[q].data = [Mb][N] out_dt,
 *         win[q].flags = [NT]: epoch once column tile j of the sum is in window q
 *
 * Supported: in BF16, slot F32 or BF16, out BF16 or F32; 1 <= Mb <= 8;
 * tile_n in {128, 256, 512}; N and K multiples of 8; Mb * N below 2^29.
 * ---------------------------------------------------------------------- */
hocf_status hocf_gemv_ar(int P, int Mb, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                         hocf_dtype out_dt, const void* x, const void* W, void* part,
                         uint32_t* part_flags, const hocf_window* win, int tile_n,
                         const hocf_sync* sync, void* stream);
size_t hocf_gemv_ar_workspace_bytes(int P, int N, int tile_n);

/* ------------------------------------------------------------------------
 * GEMV + AllReduce, unfused (the baseline the fused operator is measured
 * against: SC24's abstract compares its fused GEMV + AllReduce with running
 * the computation and then the collective).
 *
 * Same arguments, arithmetic and results as hocf_gemv_ar (the windows get
 * the same bits), computed by two kernels enqueued back to back on
 * `stream`: the GEMV, which publishes every partial into `part`, and then a
 * fold kernel (one workgroup per column tile) that folds the P partials in
 * rank order and writes the result into all P windows once the GEMV kernel
 * has ended.  Neither part_flags nor the windows' flags are written (they
 * are left as they were); part_flags must still be a valid pointer.
 * Supported combinations, limits, workspace (hocf_gemv_ar_workspace_bytes)
 * and errors as for hocf_gemv_ar.
 * ---------------------------------------------------------------------- */
hocf_status hocf_gemv_ar_unfused(int P, int Mb, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                                 hocf_dtype out_dt, const void* x, const void* W, void* part,
                                 uint32_t* part_flags, const hocf_window* win, int tile_n,
                                 const hocf_sync* sync, void* stream);

/* ------------------------------------------------------------------------
 * AllGather + GEMM.
 *
 * out = A_g . W where A_g = [chunk 0; ...; chunk P-1] (rank order).  Chunk c
 * of A_gathered (rows [c*Mc, (c+1)*Mc)) may be read only once
 * chunk_flags[c] == epoch; chunks are released in any order (by another
 * stream, a copy engine or a peer) and the kernel's workgroups claim output
 * tiles of whichever chunks have arrived.  The result does not depend on the
 * release order.  A chunk that never arrives makes the waiting workgroups
 * give up after spin_timeout_ns with HOCF_ERR_TIMEOUT.
 *
 *   A_gathered [P][Mc][K] in_dt   chunk_flags [P] (device or host-pinned)
 *   W [K][N] in_dt                out [P*Mc][N] out_dt
 *
 * Supported: in BF16, out BF16 or F32, tiles 256x256 and 128x128;
 * N and K multiples of 8.  HOCF_ERR_UNSUPPORTED when tile_m * N * (bytes
 * per output element) reaches 2^31 (an output tile's row band is stored
 * with 32-bit byte offsets).
 * ---------------------------------------------------------------------- */
hocf_status hocf_ag_gemm(int P, int Mc, int N, int K, hocf_dtype in_dt, hocf_dtype out_dt,
                         const void* A_gathered, const uint32_t* chunk_flags, const void* W,
                         void* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream);
size_t hocf_ag_gemm_workspace_bytes(int P);

/* ------------------------------------------------------------------------
 * GEMM + All-to-All (the mixture-of-experts combine).
 *
 * SC24 (abstract) names GEMM + All-to-All, for MoE layers, among its three
 * fused prototypes.  This rank holds E experts and has received token rows
 * grouped by expert: rows [expert_offsets[e], expert_offsets[e+1]) of X
 * belong to expert e, each group a whole number of tile_m-row tiles (pad a
 * group with rows whose dest is -1; their results go nowhere).  Every row i
 * is multiplied by its expert's W_e (fp32 accumulation, rounded once to
 * out_dt) and the result row is sent back to its token's rank: it lands in
 * win[dest[i]].data at row slot[i].  Tiles are scattered by the workgroup
 * that computed them while other workgroups still compute; win[d].flags[0]
 * becomes epoch once all send_counts[d] rows for destination d are there
 * (immediately, at the end of the kernel, when send_counts[d] == 0).
 *
 *   X              [T][K] in_dt (device)
 *   W              [E][K][N] in_dt (device)
 *   expert_offsets host int64 [E+1]: 0 = o_0 <= o_1 <= ... <= o_E = T, each
 *                  o_{e+1} - o_e a multiple of tile_m (read during the call)
 *   dest, slot     device int32 [T]: destination rank in [0, P) (or -1:
 *                  padding) and row in [0, cap) of each row; every (dest,
 *                  slot) pair at most once
 *   send_counts    host int64 [P]: rows with dest == d (read during the call);
 *                  each in [0, cap]
 *   win            host array of P windows; win[d].data = [cap][N] out_dt,
 *                  win[d].flags = [1]
 *
 * Supported: in BF16; tile 256x256 with out BF16 or F32, tile 128x256 with
 * out BF16; N a multiple of 256, K of 128; 1 <= E <= 64.  A row naming a destination or slot out of range
 * is skipped and HOCF_ERR_BAD_INDEX goes to the status word (that
 * destination's flag is then not set).  Rows of the windows that no row
 * names are left as they were.
 * ---------------------------------------------------------------------- */
hocf_status hocf_gemm_a2a(int P, int E, int64_t T, int N, int K, hocf_dtype in_dt, hocf_dtype out_dt,
                          const void* X, const void* W, const int64_t* expert_offsets, const int32_t* dest,
                          const int32_t* slot, const int64_t* send_counts, const hocf_window* win,
                          int64_t cap, int tile_m, int tile_n, const hocf_sync* sync, void* stream);
size_t hocf_gemm_a2a_workspace_bytes(int P);

/* ------------------------------------------------------------------------
 * All-to-All + GEMM (the mixture-of-experts dispatch, then the expert GEMM).
 *
 * The mKernel news item ("GPU-vezérelt kommunikációval gyorsítják az
 * AI-betanítást a kutatók", section on its five fused kernels) lists MoE
 * Dispatch + GEMM.  One rank's share: P source ranks each hold B tokens
 * X[p][b] ([K] each) and their router's top-k choices experts[p][b][j]
 * (global expert ids); this rank owns experts e0 .. e0+E-1.  The dispatch
 * delivers, for each local expert e in turn, the token rows of the pairs
 * (p, b, j) that chose it, in (p, b, j) order, the group padded with zero
 * rows to a multiple of tile_m; then each group is multiplied by its
 * expert's W_e (fp32 accumulation, rounded once to out_dt).  Counting,
 * prefix sums, row placement and the row copies all run on the device; an
 * expert tile starts as soon as its tile_m rows have landed, while other
 * workgroups still deliver rows.
 *
 *   X         [P][B][K] in_dt          experts  [P][B][topk] int32 (ids
 *             outside [e0, e0+E) belong to other ranks and are skipped)
 *   W         [E][K][N] in_dt
 *   recv      [cap][K] in_dt: the received rows, grouped by expert
 *   Y         [cap][N] out_dt: recv . W_e, group by group (padding rows: 0)
 *   expert_offsets  device int64 [E+1]: group e is rows [o_e, o_{e+1});
 *             o_E = rows used (a multiple of tile_m per group)
 *   dest, slot  device int32 [cap]: the source rank of each row and its
 *             position among that source's pairs landing here, in (b, j)
 *             order (-1 for padding): the routing GEMM + All-to-All takes to
 *             send each result row back
 *   send_counts device int64 [P]: each source's pairs landing here
 * Rows from o_E to cap are left as they were.  When the rows would exceed
 * cap, HOCF_ERR_CAPACITY goes to the status word, expert_offsets and
 * send_counts are written, and nothing else is.
 *
 * Supported: in BF16; tile 256x256 with out BF16 or F32, tile 128x256 with
 * out BF16; N a multiple of 256, K of 128; 1 <= E <= 64.  The workspace
 * (hocf_a2a_gemm_workspace_bytes) needs no zeroing: each call initialises
 * what it uses.  Three kernels are enqueued (counts, scans, the fused
 * dispatch + GEMM).
 * ---------------------------------------------------------------------- */
hocf_status hocf_a2a_gemm(int P, int E, int e0, int B, int topk, int N, int K, hocf_dtype in_dt, hocf_dtype out_dt,
                          const void* X, const int32_t* experts, const void* W, int64_t cap, void* recv, void* Y,
                          int64_t* expert_offsets, int32_t* dest, int32_t* slot, int64_t* send_counts, int tile_m,
                          int tile_n, const hocf_sync* sync, void* stream);
size_t hocf_a2a_gemm_workspace_bytes(int P, int E, int B, int topk, int64_t cap, int tile_m);

/* The same, unfused (the baseline): the dispatch as one kernel, then the
 * expert GEMM as the next (no tile overlaps the row delivery); the same
 * arguments and results, bit for bit. */
hocf_status hocf_a2a_gemm_unfused(int P, int E, int e0, int B, int topk, int N, int K, hocf_dtype in_dt,
                                  hocf_dtype out_dt, const void* X, const int32_t* experts, const void* W,
                                  int64_t cap, void* recv, void* Y, int64_t* expert_offsets, int32_t* dest,
                                  int32_t* slot, int64_t* send_counts, int tile_m, int tile_n,
                                  const hocf_sync* sync, void* stream);

/* ------------------------------------------------------------------------
 * Embedding bag + All-to-All.
 *
 * pooled(t, b) = sum of table t's rows listed by bag (t, b), fp32, added in
 * index order from +0.0 (an empty bag pools to zeros).  Bag b goes to
 * destination d = b / Bd (Bd = B/P), slot s = b mod Bd.
 *
 *   tables  [T][R][D] fp32
 *   indices int32: fixed-length bags [T][B][L] when offsets == NULL, else
 *           CSR: bag (t, b) = indices[offsets[t*B+b] .. offsets[t*B+b+1])
 *   offsets NULL or int64 [T*B + 1], non-decreasing, offsets[0] == 0
 *   win     host array of P windows; win[d].data = [Bd][T][D] fp32,
 *           win[d].flags = [T][NJ], NJ = ceil(Bd/tile_bags): epoch once bags
 *           [j*tile_bags, (j+1)*tile_bags) of table t are in window d
 *
 * An index outside [0, R) is skipped (the bag sums its other rows) and
 * HOCF_ERR_BAD_INDEX is recorded in *status.
 * Supported: D a multiple of 4 up to 512; B % P == 0; tile_bags in [1, 4096]
 *            with tile_bags * T * D * 4 < 2^31 (else HOCF_ERR_UNSUPPORTED).
 * ---------------------------------------------------------------------- */
hocf_status hocf_embbag_a2a(int T, int64_t R, int D, int B, int L, int P, const float* tables,
                            const int32_t* indices, const int64_t* offsets,
                            const hocf_window* win, int tile_bags, const hocf_sync* sync,
                            void* stream);
size_t hocf_embbag_a2a_workspace_bytes(void);

/* ------------------------------------------------------------------------
 * Point-to-point puts, optionally with a completion signal, on the copy
 * engines.
 *
 * HOCCL (abstract) drives collective communication with the GPU's DMA
 * engines so that no compute unit takes part in moving the data, and keeps
 * that traffic in order with the compute kernels through their streams.
 * hocf_dma_put is that point-to-point step: for i = 0 .. n-1, in order on
 * `stream`, it copies bytes[i] bytes from src[i] to dst[i] and then, if
 * signal and signal[i] are non-NULL, copies the 32-bit word at signal_value
 * to signal[i].  Each copy starts once the one before it has completed.
 *
 * Two ways to consume the bytes:
 *   - in stream order (HOCCL's operator-level ordering): work enqueued after
 *     an event recorded on `stream` behind the puts sees them;
 *   - while they land: a kernel running on another stream (e.g. hocf_ag_gemm
 *     with signal[i] = &chunk_flags[c] and *signal_value = its epoch) that
 *     sees signal[i] equal to *signal_value after a system-scope acquire
 *     sees all of dst[i].
 *
 *   engine HOCF_ENGINE_DMA   copies on a copy (SDMA) engine, no compute unit;
 *                            but the HIP runtime runs any copy below 64 KB,
 *                            so every signal, as a one-workgroup copy kernel
 *                            of a few microseconds, which waits for a free
 *                            CU (a kernel holding every CU delays it, and
 *                            the puts after it, until it ends)
 *          HOCF_ENGINE_CU    the same copies as the runtime's copy kernels,
 *                            which occupy compute units (the comparison)
 *   src, dst, bytes          host arrays of n entries; src[i], dst[i]
 *                            16-byte aligned device memory of the current
 *                            device (may be NULL when bytes[i] == 0)
 *   signal                   NULL (no put signals), or a host array of n
 *                            pointers, each NULL (no signal for that put) or
 *                            a 4-byte aligned device word
 *   signal_value             device word, 4-byte aligned, holding the value
 *                            to publish when the stream reaches the puts
 *                            (ignored when no put signals)
 *
 * 0 <= n <= HOCF_MAX_PUTS.  Every dst range and signal word is written and
 * may overlap no other range of the call (HOCF_ERR_INVALID_ARG), as may a
 * pointer the runtime does not know as device memory of the current device.
 * A copy the runtime refuses returns HOCF_ERR_HIP; the puts before it stay
 * enqueued.  Nothing is allocated; the caller owns every buffer and must
 * keep src and signal_value unchanged until the stream has passed the puts.
 * ---------------------------------------------------------------------- */
#define HOCF_MAX_PUTS 16
typedef enum hocf_engine HOCF_ENUM_INT { HOCF_ENGINE_DMA = 0, HOCF_ENGINE_CU = 1 } hocf_engine;
hocf_status hocf_dma_put(int n, const void* const* src, void* const* dst, const int64_t* bytes,
                         uint32_t* const* signal, const uint32_t* signal_value, hocf_engine engine,
                         void* stream);

/* ---------------------------------------------------------------------- */
const char* hocf_status_string(hocf_status s); /* static string, never NULL */
const char* hocf_last_error(void);             /* detail of this thread's last error */
int hocf_abi_version(void);                    /* HOCF_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif /* HOCF_H */
