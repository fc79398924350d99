// GEMM + ReduceScatter, fused in one persistent kernel.
//
// mKernel news item ("GPU-vezérelt kommunikációval gyorsítják az
// AI-betanítást a kutatók"): GEMM + ReduceScatter is one of its five fused
// kernels, with communication in the same persistent kernel as the compute
// and tile-level overlap.  SC24 ("Optimizing Distributed ML Communication
// with Fused Computation-Collective Operations", abstract): each workgroup
// sends its result on as soon as its computation is done while the other
// workgroups of the kernel keep computing.
//
// Work item = one TM x TN tile of one shard's partial C_p = A_p . W_p.
// Items are dealt from eight ticket queues, one per XCD: queue q holds a
// contiguous range of the item list ordered (p, chunk r, column tile, row
// tile), so with P = 8 an XCD computes one shard and its 32 concurrent
// tiles share A row panels and W column panels in that XCD's L2.
//
// When a tile is done the workgroup
//   1. stores it into destination r's window, slot p (publish), with
//      device-coherent full-row stores, and waits for their completion,
//   2. stores the epoch into the tile's ready flag in window r,
//   3. counts itself in the output tile's arrival counter (an atomic add
//      whose result it does not wait for); the tile is ready once the count
//      reaches P: its reduction is PIECES bands of rows, band q of every
//      output tile sitting in band queue q (one queue per XCD),
//   4. folds one band of a completed tile, if its band queue has one for it:
//      checks the P flags and folds the P slots of the band's rows in rank
//      order p = 0..P-1 in fp32 into the destination's output chunk -- while
//      other workgroups are still computing.  Where the tile shape allows,
//      the band rides along the workgroup's next GEMM tile: one row pass of
//      slot loads is issued at the end of each K round of the mainloop and
//      folded at the end of the next, so the band's memory latency hides
//      behind MFMA work instead of stalling the workgroup.
// With P = PIECES every workgroup alternates one GEMM tile and one band, so
// the reduction traffic is spread evenly and the workgroups of an XCD stay in
// step, which keeps their shared operand panels in L2.  The slots of a band
// queue follow the order in which output tiles complete (every shard's
// items run in the same chunk and tile order), so a workgroup claims the
// next slot of its home queue with one atomic add, holds it, and checks its
// tile's arrival count after each of its own tiles, never waiting while
// tiles remain.  The last workgroup out zeroes the counts for the next call.
// Without tiles a workgroup waits (bounded) for its slot, then helps drain
// the other queues; tiles are always claimed by running workgroups, so
// every slot becomes ready and the kernel ends.
// No step needs an L2-wide write-back or invalidate (publish.hpp).
#include <mutex>
#include <type_traits>
#include <unordered_map>
#include <vector>

#include "internal.hpp"
#include "mfma_tile.hpp"
#include "publish.hpp"
#include "sync.hpp"
#include "trace.hpp"

namespace hocf {

// Where band `piece` of completed output tile `g` (group = (chunk r, tile))
// lives: its tile in slot 0 of window r, its output rows, and the flags that
// announced the tile's P contributions.
template <class Tile, int SDT, int ODT>
struct BandRef {
  const char* slot0;
  int64_t slot_bytes;
  int64_t otile_off;  // byte offset of the band's output tile in every output
  int row0, rows_valid, cols_valid;
  const uint32_t* flags;  // flag of contribution q at flags[q * tiles per chunk]

  __device__ __forceinline__ BandRef(const GemmRsArgs& a, int64_t g, int piece) {
    using RL = ReduceLayout<Tile, SDT>;
    constexpr int SES = SDT == kBF16 ? 2 : 4;
    const int N = a.N, Mc = a.Mc;
    const int tpc = a.mtiles * a.ntiles;
    const int r = (int)(g / tpc), tflag = (int)(g % tpc);
    const int mt = tflag / a.ntiles, nt = tflag % a.ntiles;
    rows_valid = min(Tile::TM, Mc - mt * Tile::TM);
    cols_valid = min(Tile::TN, a.Nc - nt * Tile::TN);
    row0 = piece * RL::PIECE_ROWS;
    const int64_t tile_off = (int64_t)mt * Tile::TM * N + (int64_t)nt * Tile::TN;
    slot0 = reinterpret_cast<const char*>(a.win_data[r]) + tile_off * SES;
    slot_bytes = (int64_t)Mc * N * SES;
    otile_off = ((int64_t)r * Mc * N + tile_off) * (ODT == kBF16 ? 2 : 4);
    flags = &a.win_flags[r][tflag];
  }
  // the P contributions' flags must all carry this call's epoch (one thread
  // each): the flag this thread checks (the epoch itself for threads >= P) ...
  __device__ __forceinline__ uint32_t my_flag(const GemmRsArgs& a, int tpc) const {
    return (int)threadIdx.x < a.P ? load_flag_agent(&flags[(int64_t)threadIdx.x * tpc]) : a.sync.epoch;
  }
  // ... and the check, which may come later than the load (a producer does
  // not wait for its flag store before counting itself, so a flag read
  // early is read again, bounded, before it counts as missing)
  __device__ __forceinline__ void verify(const GemmRsArgs& a, int tpc, uint32_t flag) const {
    if ((int)threadIdx.x < a.P) expect_flag(&flags[(int64_t)threadIdx.x * tpc], flag, a.sync);
  }
  __device__ __forceinline__ void check_flags(const GemmRsArgs& a, int tpc) const {
    verify(a, tpc, my_flag(a, tpc));
  }
  // the outputs the band goes to: the first `n` of a.outs
  __device__ __forceinline__ OutSet outs(const GemmRsArgs& a, int n) const { return OutSet{a.outs, n, otile_off}; }
};

// Folds band `piece` of completed output tile `g` on its own, into the
// first `nout` outputs (checking the P contributions' flags first, unless
// the partials are known complete: the unfused fold kernel).
template <class Tile, bool RAGGED, int SDT, int ODT, bool CHECK = true>
__device__ __forceinline__ void reduce_band(const GemmRsArgs& a, int64_t g, int piece, int nout) {
  const BandRef<Tile, SDT, ODT> b(a, g, piece);
  if (RAGGED && b.row0 >= b.rows_valid) return;
  if constexpr (CHECK) b.check_flags(a, a.mtiles * a.ntiles);
  const int P = a.P, N = a.N;
  if (P <= 4)
    reduce_piece<Tile, SDT, ODT, RAGGED, 4, 8>(b.slot0, b.slot_bytes, P, N, b.outs(a, nout), N, b.row0, b.rows_valid,
                                               b.cols_valid);
  else if (P <= 8)
    reduce_piece<Tile, SDT, ODT, RAGGED, 8, 4>(b.slot0, b.slot_bytes, P, N, b.outs(a, nout), N, b.row0, b.rows_valid,
                                               b.cols_valid);
  else
    reduce_piece<Tile, SDT, ODT, RAGGED, kMaxP, 2>(b.slot0, b.slot_bytes, P, N, b.outs(a, nout), N, b.row0,
                                                   b.rows_valid, b.cols_valid);
}

// What the kernel body does with a finished tile.
enum GemmMode {
  kFusedRS = 0,  // GEMM + ReduceScatter: publish, flag, fold bands into the one output
  kFusedAR = 1,  // GEMM + AllReduce: the same, each folded band stored to all a.nout windows
  kGemmOnly = 2  // the unfused baseline's first kernel: publish the tile, nothing else
};

// The kernel body shared by the fused operators and the unfused baseline's
// GEMM kernel (MODE above).
template <class Tile, bool RAGGED, bool BF16IN, int SDT, int ODT, int MODE>
__device__ __forceinline__ void gemm_collective(const GemmRsArgs& a) {
  constexpr bool AR = MODE == kFusedAR, FUSED = MODE != kGemmOnly;
  using Elem = typename std::conditional<BF16IN, uint16_t, float>::type;
  constexpr int S = ReduceLayout<Tile, SDT>::PIECES;
  // tiles with a split mainloop start the next tile's loads before the band
  constexpr bool kSplit = Tile::kSplitMainloop;
  // ... and, if the band's parked rows fit in LDS beside the stages, fold the
  // band during the tile's mainloop (full tiles, P <= 8, enough K rounds)
  using Band = BandFold<Tile, SDT, ODT, 8>;
  constexpr bool kBandInLoop = kSplit && !RAGGED && Tile::LDS_BYTES + Band::LDS_BYTES + 1024 <= 160 * 1024;
  __shared__ __attribute__((aligned(16))) char band_park[kBandInLoop ? Band::LDS_BYTES : 16];
  // LDS stages, one __shared__ array each (tiles with fewer stages leave the rest tiny)
  __shared__ __attribute__((aligned(1024))) char smem0[Tile::SMEM_BYTES];
  __shared__ __attribute__((aligned(1024))) char smem1[Tile::NST > 1 ? Tile::SMEM_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char smem2[Tile::NST > 2 ? Tile::SMEM_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char smem3[Tile::NST > 3 ? Tile::SMEM_BYTES : 16];
  char* const stages[4] = {smem0, smem1, smem2, smem3};
  __shared__ int64_t s_item;
  __shared__ int s_last;
  __shared__ int s_band, s_state;

  const int tid = threadIdx.x;
  const int P = a.P, N = a.N, K = a.K, Mc = a.Mc;
  const int nout = AR ? a.nout : 1;
  const int tpc = a.mtiles * a.ntiles;
  const int64_t ngroups = (int64_t)P * tpc;
  // workspace after the queue block: arrival counters [P][tpc] (an output
  // tile is ready when its count reaches P), band queue heads [8] (and 8
  // spare words), then one spare word per output tile
  uint32_t* grp = a.ws + kWsExtra;
  uint32_t* bq_head = grp + ngroups;
  // Band queue q (q < S) holds band q of every output tile, in the order in
  // which the tiles' last contributions are computed (chunk-major, then the
  // item order within a chunk): slot t -> output tile band_tile(t).  A slot
  // is claimed with one atomic add on the queue's head and is ready once
  // its tile's arrival count is P; producers never touch the queues.
  auto bq_total = [&](int q) { return q < S ? (uint32_t)ngroups : 0u; };
  auto band_tile = [&](uint32_t t) {
    const int r = (int)(t / tpc), tq = (int)(t % tpc);
    return (int64_t)r * tpc + (int64_t)(tq % a.mtiles) * a.ntiles + tq / a.mtiles;
  };
  const int home = (int)(blockIdx.x % kNumQueues) % S;
  constexpr int SES = SDT == kBF16 ? 2 : 4;
  bool loop_band_ok = false;
  if constexpr (kBandInLoop)
    loop_band_ok = P <= 8 && Tile::side_fits(K, Band::NPASS) && (int64_t)P * Mc * N * SES < (int64_t(1) << 31);

  // thread 0's claim state: tiles and band slots are both requested one
  // iteration ahead; a claimed band slot (queue, index) waits in pend_* until
  // its band has been handed out
  ClaimAhead tiles;
  TraceSink trace;
  trace.init(a.trace);
  int pend_q = -1;
  uint32_t pend_i = 0;
  bool band_ahead = false;
  uint32_t band_ticket = 0;
  bool tiles_left = true;
  for (;;) {
    // the next tile, and a band of a completed tile to fold in this
    // iteration if one is ready (one thread-0 region between two barriers)
    trace.mark(kTrStart);
    __syncthreads();
    if (tid == 0 && !FUSED) {
      // unfused: tiles only; the folds are a separate kernel
      const int64_t it = tiles_left ? tiles.next(a.ws, a.total) : -1;
      s_item = it;
      s_state = it >= 0 ? 0 : 2;
      s_band = -1;
    } else if (tid == 0) {
      const int64_t it = tiles_left ? tiles.next(a.ws, a.total) : -1;
      const bool tl = it >= 0;
      int state = 0;  // 0: none now, 1: band ready, 2: all bands taken, 3: timed out
      int band = -1;
      if (band_ahead) {
        if (band_ticket < bq_total(home)) { pend_q = home; pend_i = band_ticket; }
        band_ahead = false;
      }
      if (pend_q < 0) {
        // claim a slot: the home queue while tiles remain, any queue after
        for (int i = 0; i < (tl ? 1 : kNumQueues); ++i) {
          const int q = (home + i) % kNumQueues;
          if (__hip_atomic_load(&bq_head[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= bq_total(q)) continue;
          const uint32_t t = __hip_atomic_fetch_add(&bq_head[q], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (t < bq_total(q)) { pend_q = q; pend_i = t; break; }
        }
        if (pend_q < 0 && !tl) state = 2;
      }
      if (pend_q >= 0) {
        const int64_t g = band_tile(pend_i);
        uint32_t e = __hip_atomic_load(&grp[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)P;
        if (e == 0 && !tl) {
          // nothing else to do: wait (bounded; an abort request ends it) for
          // the slot's tile to complete
          const Deadline wl{now_ticks(), a.sync.timeout_ticks};
          int w = kWaitOk;
          while (e == 0) {
            __builtin_amdgcn_s_sleep(4);
            e = __hip_atomic_load(&grp[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)P;
            if (e != 0) break;
            if (abort_requested(a.sync)) { w = kWaitAborted; break; }
            if (wl.expired()) { w = kWaitTimeout; break; }
          }
          if (e == 0) { report_wait(a.sync, w); state = 3; }
        }
        if (e != 0) {
          band = (int)(g * S + pend_q);
          state = 1;
          pend_q = -1;
          if (tl) {
            // the next slot of the home queue, its result read next iteration
            band_ticket = __hip_atomic_fetch_add(&bq_head[home], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            band_ahead = true;
          }
        }
      }
      s_item = it;
      s_state = state;
      s_band = band;
    }
    __syncthreads();
    const int64_t item = uniform64(s_item);
    const int state = uniform(s_state);
    const int band = uniform(s_band);
    trace.mark(kTrClaimed);
    if (item < 0) tiles_left = false;
    if (item < 0 && state != 1) {
      if (state >= 2 || !tiles_left) break;  // all bands taken, or a timeout was reported
      continue;
    }

    int r = 0, p = 0, tflag = 0, mt = 0, nt = 0;
    const Elem* At = nullptr;
    const Elem* Wt = nullptr;
    if (item >= 0) {
      const int tq = (int)(item % tpc);
      r = (int)((item / tpc) % P);
      p = (int)(item / ((int64_t)tpc * P));
      nt = tq / a.mtiles;
      mt = tq % a.mtiles;
      tflag = mt * a.ntiles + nt;
      At = reinterpret_cast<const Elem*>(a.A) + ((int64_t)p * a.M + (int64_t)r * Mc + (int64_t)mt * Tile::TM) * K;
      Wt = reinterpret_cast<const Elem*>(a.W) + (int64_t)p * K * N + (int64_t)nt * Tile::TN;
    }
    // 4. the band: folded during this iteration's mainloop, or on its own
    // while the tile's first operand slices load (it does not touch the stages)
    const bool band_in_loop = kBandInLoop && loop_band_ok && state == 1 && item >= 0;
    // (the in-loop band's flags are loaded now and checked after the mainloop)
    uint32_t band_flag = 0;
    if (band_in_loop) band_flag = BandRef<Tile, SDT, ODT>(a, band / S, band % S).my_flag(a, tpc);
    if (item >= 0) {
      if constexpr (kSplit) Tile::prologue(At, K, Wt, N, K, stages);
    }
    if (state == 1 && !band_in_loop) reduce_band<Tile, RAGGED, SDT, ODT>(a, band / S, band % S, nout);
    trace.mark(kTrMainStart);

    if (item >= 0) {
      const int rows_valid = min(Tile::TM, Mc - mt * Tile::TM);
      const int cols_valid = min(Tile::TN, a.Nc - nt * Tile::TN);
      floatx16 acc[Tile::FM][Tile::FN];
      if constexpr (kBandInLoop) {
        if (band_in_loop) {
          const BandRef<Tile, SDT, ODT> b(a, band / S, band % S);
          Band side;
          side.init(b.slot0, (uint32_t)b.slot_bytes, P, N, b.row0,
                    (typename Band::lds_char*)(band_park));
          Tile::template body_side<RAGGED>(At, K, Wt, N, rows_valid, cols_valid, K, stages, acc, side);
          side.flush(b.outs(a, nout), N, b.row0);
          b.verify(a, tpc, band_flag);
        } else {
          Tile::template body<RAGGED>(At, K, Wt, N, rows_valid, cols_valid, K, stages, acc);
        }
      } else if constexpr (kSplit) {
        Tile::template body<RAGGED>(At, K, Wt, N, rows_valid, cols_valid, K, stages, acc);
      } else {
        Tile::template run<RAGGED>(At, K, Wt, N, rows_valid, cols_valid, K, stages, acc);
      }

      trace.mark(kTrMainEnd);

      // 1. publish the tile into window r, slot p
      char* wdata = reinterpret_cast<char*>(a.win_data[r]);
      const int64_t tile_off = (int64_t)mt * Tile::TM * N + (int64_t)nt * Tile::TN;
      store_tile<Tile, SDT, RAGGED, kPolicyDevice, false>(wdata + ((int64_t)p * Mc * N + tile_off) * SES, N,
                                                          rows_valid, cols_valid, acc, stages);
    }

    uint32_t completed = 0;  // (thread 0, trace build only)
    if (FUSED && item >= 0) {
      wait_memory();  // this thread's stores of the tile have completed
      __syncthreads();
      trace.mark(kTrStored);
      // 2. ready flag; 3. arrival count (P: the tile's bands are ready)
      if (tid == 0) {
        // (the tile's data is complete; readers of the flag re-read it, bounded,
        // if they get there before the flag store has)
        __hip_atomic_store(&a.win_flags[r][(int64_t)p * tpc + tflag], a.sync.epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        // (no wait for the result: a band's claimer reads the count itself;
        // only the trace build looks at it, to mark the tile's completion)
        const uint32_t prev =
            __hip_atomic_fetch_add(&grp[(int64_t)r * tpc + tflag], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (kTraceBuild) {
          if (prev == (uint32_t)(P - 1)) completed = kTrCompleted;
        }
      }
      // (the barrier at the top of the loop ends this thread-0 region)
    }
    if constexpr (kTraceBuild) {
      trace.mark(kTrDone);
      trace.commit(item, state == 1 ? band : -1,
                   completed | (state == 1 ? (band_in_loop ? kTrBandInLoop : kTrBandAlone) : 0u));
    }
  }

  // the last workgroup out leaves the workspace zeroed (arrival counts, queue
  // heads and the spare words after them)
  if (finish_workgroup_last(a.ws, &s_last)) {
    for (int64_t i = tid; i < ngroups + 2 * kNumQueues + ngroups; i += Tile::NT)
      __hip_atomic_store(&grp[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <class Tile, bool RAGGED, bool BF16IN, int SDT, int ODT>
__global__ __launch_bounds__(Tile::NT) void gemm_rs_kernel(GemmRsArgs a) {
  gemm_collective<Tile, RAGGED, BF16IN, SDT, ODT, kFusedRS>(a);
}

template <class Tile, bool RAGGED, bool BF16IN, int SDT, int ODT>
__global__ __launch_bounds__(Tile::NT) void gemm_ar_kernel(GemmRsArgs a) {
  gemm_collective<Tile, RAGGED, BF16IN, SDT, ODT, kFusedAR>(a);
}

// The unfused baseline: the same GEMM, every tile published into its slot and
// nothing else (no flags, no counts, no folds) ...
template <class Tile, bool RAGGED, bool BF16IN, int SDT, int ODT>
__global__ __launch_bounds__(Tile::NT) void unfused_gemm_kernel(GemmRsArgs a) {
  gemm_collective<Tile, RAGGED, BF16IN, SDT, ODT, kGemmOnly>(a);
}

// ... then, once that kernel has ended (stream order), one workgroup per band
// of every output tile folds the P slots in rank order into the output.
template <class Tile, bool RAGGED, int SDT, int ODT>
__global__ __launch_bounds__(Tile::NT) void unfused_fold_kernel(GemmRsArgs a) {
  constexpr int S = ReduceLayout<Tile, SDT>::PIECES;
  reduce_band<Tile, RAGGED, SDT, ODT, false>(a, (int64_t)blockIdx.x / S, (int)(blockIdx.x % S), 1);
}

template <class Tile, bool RAGGED, bool BF16IN, int SDT, int ODT>
static int launch_one(const GemmRsArgs& a, hipStream_t s) {
  auto kern = a.mode == kFusedAR ? &gemm_ar_kernel<Tile, RAGGED, BF16IN, SDT, ODT>
            : a.mode == kGemmOnly ? &unfused_gemm_kernel<Tile, RAGGED, BF16IN, SDT, ODT>
                                  : &gemm_rs_kernel<Tile, RAGGED, BF16IN, SDT, ODT>;
  // the fold kernel of the unfused form: P chunks x tiles per chunk x bands per tile workgroups
  const int64_t folds = (int64_t)a.P * a.mtiles * a.ntiles * ReduceLayout<Tile, SDT>::PIECES;
  if (a.mode == kGemmOnly && folds > 0x7FFFFFFF) return kNoKernel;
  int grid = 0;
  hipError_t e = persistent_grid(reinterpret_cast<const void*>(kern), Tile::NT, a.total, &grid, a.max_wg);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Tile::NT), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.mode != kGemmOnly) return e;
  hipStream_t fs = s;
  if (a.fold_stream) {
    fs = static_cast<hipStream_t>(a.fold_stream);
    if ((e = hipEventRecord(static_cast<hipEvent_t>(a.gemm_done), s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(fs, static_cast<hipEvent_t>(a.gemm_done), 0)) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((unfused_fold_kernel<Tile, RAGGED, SDT, ODT>), dim3((unsigned)folds), dim3(Tile::NT), 0, fs,
                     a);
  return hipGetLastError();
}

template <class Tile, bool BF16IN, int SDT, int ODT>
static int launch_tile(const GemmRsArgs& a, hipStream_t s) {
  const bool ragged = (a.Mc % Tile::TM) || (a.Nc % Tile::TN) || (a.K % Tile::BK);
  return ragged ? launch_one<Tile, true, BF16IN, SDT, ODT>(a, s)
                : launch_one<Tile, false, BF16IN, SDT, ODT>(a, s);
}

// bf16: full tiles take the direct-to-LDS mainloop, ragged ones the
// register-staged mainloop that zero-fills the edges
template <int TM, int TN, int SDT, int ODT>
static int launch_bf16_dt(const GemmRsArgs& a, hipStream_t s) {
  using Staged = TileBf16<TM, TN, 2, 2>;
  using Direct = TileBf16Direct<TM, TN, 2, 2>;
  // the direct tile takes full tiles whose operands it can address with 32-bit offsets
  const bool ragged = (a.Mc % TM) || (a.Nc % TN) || !Direct::k_fits(a.K) ||
                      !Direct::operands_fit(a.K, a.N, a.K);
  return ragged ? launch_one<Staged, true, true, SDT, ODT>(a, s)
                : launch_one<Direct, false, true, SDT, ODT>(a, s);
}

template <int TM, int TN>
static int launch_bf16(const GemmRsArgs& a, hipStream_t s) {
  if (a.slot_dt == kF32 && a.out_dt == kBF16) return launch_bf16_dt<TM, TN, kF32, kBF16>(a, s);
  if (a.slot_dt == kBF16 && a.out_dt == kBF16) return launch_bf16_dt<TM, TN, kBF16, kBF16>(a, s);
  if (a.slot_dt == kF32 && a.out_dt == kF32) return launch_bf16_dt<TM, TN, kF32, kF32>(a, s);
  if (a.slot_dt == kBF16 && a.out_dt == kF32) return launch_bf16_dt<TM, TN, kBF16, kF32>(a, s);
  return kNoKernel;
}

int launch_gemm_rs(const GemmRsArgs& a, int tm, int tn, int in_dt, hipStream_t s) {
  if (in_dt == kBF16) {
    if (tm == 256 && tn == 256) return launch_bf16<256, 256>(a, s);
    if (tm == 128 && tn == 128) return launch_bf16<128, 128>(a, s);
  } else if (a.slot_dt == kF32 && a.out_dt == kF32) {
    if (tm == 64 && tn == 64) return launch_tile<TileF32<64, 64, 2, 2>, false, kF32, kF32>(a, s);
  }
  return kNoKernel;
}

// ------------------------------------------------------------------------
// The decomposed form (Compass, abstract: inter-operator decomposition, a
// tensor split into parts whose computation and communication are
// pipelined).  Piece i is columns [i*N/pieces, (i+1)*N/pieces) of every
// partial and of the output: its shard GEMMs (the unfused GEMM kernel, the
// grid capped to leave fold_cus CUs free) run on s, an event marks their
// end, and its fold runs on coll after that event -- while piece i+1's
// GEMMs run on s.  At the end s waits for coll's last fold.  The events are
// kept per host thread and device (created at first use, reused by every
// later call of that thread).
static hipError_t piece_events(hipEvent_t** out) {
  // per host thread and device: a call records and waits on its events in
  // order, so another thread's call cannot record one of them in between
  thread_local std::unordered_map<int, std::vector<hipEvent_t>> ev;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::vector<hipEvent_t>& v = ev[dev];
  while (v.size() < (size_t)kMaxPieces + 1) {
    hipEvent_t x = nullptr;
    if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) return e;
    v.push_back(x);
  }
  *out = v.data();
  return hipSuccess;
}

int launch_gemm_rs_pieces(const GemmRsArgs& a0, int tm, int tn, int in_dt, int pieces, int fold_cus,
                          hipStream_t s, hipStream_t coll) {
  if (pieces < 1 || pieces > kMaxPieces || a0.N % pieces || (a0.N / pieces) % tn) return kNoKernel;
  hipEvent_t* ev = nullptr;
  hipError_t e = piece_events(&ev);
  if (e != hipSuccess) return e;
  DeviceInfo di;
  if ((e = device_info(&di)) != hipSuccess) return e;
  const int ses = a0.slot_dt == kBF16 ? 2 : 4, oes = a0.out_dt == kBF16 ? 2 : 4, ies = in_dt == kBF16 ? 2 : 4;
  const int w = a0.N / pieces;
  for (int i = 0; i < pieces; ++i) {
    GemmRsArgs a = a0;
    const int64_t c0 = (int64_t)i * w;
    a.W = static_cast<const char*>(a0.W) + c0 * ies;
    for (int r = 0; r < a.P; ++r) a.win_data[r] = static_cast<char*>(a0.win_data[r]) + c0 * ses;
    a.outs[0] = static_cast<char*>(a0.outs[0]) + c0 * oes;
    a.Nc = w;
    a.ntiles = w / tn;
    a.total = (int64_t)a.P * a.P * a.mtiles * a.ntiles;
    a.mode = kGemmOnly;
    a.max_wg = fold_cus > 0 && fold_cus < di.cus ? di.cus - fold_cus : 0;
    a.fold_stream = coll;
    a.gemm_done = ev[i];
    const int r = launch_gemm_rs(a, tm, tn, in_dt, s);
    if (r != hipSuccess) return r;
  }
  if ((e = hipEventRecord(ev[kMaxPieces], coll)) != hipSuccess) return e;
  return hipStreamWaitEvent(s, ev[kMaxPieces], 0);
}

// ------------------------------------------------------------------------
// Scratch of the entry point that allocates nothing (hocf_gemm_rs_noalloc):
// the scheduler words a caller's workspace holds otherwise, in a file-scope
// device array.  Each device the library runs on holds its own copy until
// the process ends; every no-allocation call on a device shares it, so such
// calls must not overlap on one device.  In host code `scratch` names a
// host-side stand-in, never the device memory: kernels receive the address
// noalloc_scratch() obtained from the runtime for the current device.
static __device__ __align__(256) uint32_t scratch[kNoAllocScratchBytes / 4];

hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static std::unordered_map<int, void*> addr;  // device -> its copy of `scratch`
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    // (once per device, with that device current)
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    it = addr.emplace(dev, p).first;
  }
  *out = it->second;
  return hipSuccess;
}

// Zeroes n words at p: a kernel, not a memset, so that a caller may capture
// the call in a HIP graph.
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

int launch_zero_words(uint32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace hocf
