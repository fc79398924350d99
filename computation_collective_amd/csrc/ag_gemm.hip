// AllGather + GEMM with chunk-gated tile claiming.
//
// mKernel news item ("GPU-vezérelt kommunikációval gyorsítják az
// AI-betanítást a kutatók"): AllGather + GEMM is one of its five fused
// kernels, overlapping the arriving chunks with compute at tile/chunk
// granularity inside one persistent kernel.
//
// Chunk c of the gathered A (rows [c*Mc, (c+1)*Mc)) is written by someone
// else -- a copy engine, another stream, a peer -- which then sets
// chunk_flags[c] = epoch.  Chunks are served in arrival order: the first
// workgroup that sees a chunk's flag appends the chunk to an arrival list in
// the workspace.  Tiles are dealt from one ticket counter: ticket t is tile
// (t mod Tc) of the chunk at arrival position (t / Tc), Tc = tiles per chunk,
// so a workgroup that draws a ticket waits (bounded) only for the chunk its
// ticket names, and never for another workgroup.  A workgroup whose chunk is
// already on the list only acquires it (no flag polling, no atomic on the
// registration mask); otherwise it polls all flags with one batch of loads
// and acquires (system scope: the writer may be a DMA engine) once per batch
// of newly seen chunks, before it reads any of them.  Tiles are computed identically whatever the order, so the output
// does not depend on the release order.
//
// Every wait is bounded: after the time limit (or an abort request) the
// waiting workgroup records the error and exits, so the kernel always ends.
//
// Workspace words after the common queue block (kWsExtra):
//   0           ticket counter (tickets from gridDim.x on)
//   1           mask of chunks already appended to the arrival list
//   2           (unused)
//   [3, 3+P)    arrival list (chunk id + 1)
//   3 + P       count of finished workgroups (the last one resets all words)
#include "internal.hpp"
#include "mfma_tile.hpp"
#include "publish.hpp"
#include "sync.hpp"

namespace hocf {

template <class Tile, bool RAGGED, int ODT>
__global__ __launch_bounds__(Tile::NT) void ag_gemm_kernel(AgGemmArgs a) {
  // LDS stages, one __shared__ array each (tiles with fewer stages leave the rest tiny)
  __shared__ __attribute__((aligned(1024))) char smem0[Tile::SMEM_BYTES];
  __shared__ __attribute__((aligned(1024))) char smem1[Tile::NST > 1 ? Tile::SMEM_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char smem2[Tile::NST > 2 ? Tile::SMEM_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char smem3[Tile::NST > 3 ? Tile::SMEM_BYTES : 16];
  char* const stages[4] = {smem0, smem1, smem2, smem3};
  __shared__ int s_chunk, s_tile;

  const int tid = threadIdx.x;
  const int P = a.P, N = a.N, K = a.K, Mc = a.Mc;
  const int tpc = a.mtiles * a.ntiles;
  uint32_t* ws = a.ws + kWsExtra;
  uint32_t* ticket = ws;
  uint32_t* reg_mask = ws + 1;
  uint32_t* arr = ws + 3;
  uint32_t* done = ws + 3 + P;
  const uint32_t total = (uint32_t)P * (uint32_t)tpc;

  // thread 0's private state
  uint32_t seen = 0;  // chunks whose flag this workgroup has acquired
  Deadline dl{now_ticks(), a.sync.timeout_ticks};

  bool first = true;
  for (;;) {
    __syncthreads();  // keeps the thread-0 claim region apart from the previous iteration
    if (tid == 0) {
      int chunk = -1, tile = -1;
      // the first gridDim.x tickets go to the workgroups by index (no
      // atomic: at the start every workgroup would hit the counter at once),
      // each XCD's workgroups taking a contiguous run of them (tiles of the
      // same chunk share its A rows in that XCD's L2); the counter deals the
      // tickets after them
      const uint32_t tk = first ? xcd_contiguous(blockIdx.x, gridDim.x)
                                : gridDim.x + __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED,
                                                                     __HIP_MEMORY_SCOPE_AGENT);
      first = false;
      if (tk < total) {
        const uint32_t pos = tk / (uint32_t)tpc;
        dl.start = now_ticks();  // the bound is per wait
        for (;;) {
          // one batch of loads: the arrival list entry for this ticket and
          // every flag not yet seen by this workgroup
          const uint32_t e = __hip_atomic_load(&arr[pos], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          uint32_t fv[kMaxP];
#pragma unroll
          for (int q = 0; q < kMaxP; ++q)
            if (q < P && !(seen & (1u << q))) fv[q] = load_flag_system(&a.chunk_flags[q]);
          // 1. the chunk at this ticket's arrival position, once someone has
          //    registered it (after seeing its flag): acquired by this
          //    workgroup before any of its rows is read
          if (e != 0) {
            const int q = (int)e - 1;
            if (!(seen & (1u << q))) {
              acquire_system();
              seen |= 1u << q;
            }
            chunk = q;
            tile = (int)(tk % (uint32_t)tpc);
            break;
          }
          // 2. not registered yet: the newly arrived chunks, acquired at once;
          //    the ones nobody registered yet go on the arrival list.  One
          //    atomic OR on the registration mask orders registrations: the
          //    chunks this one adds take the next positions after those
          //    already registered (popcount of the old mask), in index order.
          uint32_t fresh = 0;
#pragma unroll
          for (int q = 0; q < kMaxP; ++q)
            if (q < P && !(seen & (1u << q)) && fv[q] == a.sync.epoch) fresh |= 1u << q;
          if (fresh) {
            acquire_system();
            seen |= fresh;
            const uint32_t old = __hip_atomic_fetch_or(reg_mask, fresh, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t mine = fresh & ~old;
            uint32_t at = (uint32_t)__builtin_popcount(old);
            for (int q = 0; q < P; ++q) {
              if (!(mine & (1u << q))) continue;
              __hip_atomic_store(&arr[at], (uint32_t)q + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if (at == pos) { chunk = q; tile = (int)(tk % (uint32_t)tpc); }
              ++at;
            }
            if (chunk >= 0) break;  // this workgroup registered its own ticket's chunk
            continue;               // look at the arrival list again
          }
          // 3. not there yet: bounded wait
          if (abort_requested(a.sync)) {
            report_status(a.sync, kErrAborted);
            break;
          }
          if (dl.expired()) {
            report_status(a.sync, kErrTimeout);
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
      }
      s_chunk = chunk;
      s_tile = tile;
    }
    __syncthreads();
    const int c = uniform(s_chunk), t = uniform(s_tile);
    __syncthreads();
    if (c < 0) break;

    const int nt = t / a.mtiles, mt = t % a.mtiles;
    const int rows_valid = min(Tile::TM, Mc - mt * Tile::TM);
    const int cols_valid = min(Tile::TN, N - nt * Tile::TN);
    const uint16_t* At = a.A + ((int64_t)c * Mc + (int64_t)mt * Tile::TM) * K;
    const uint16_t* Wt = a.W + (int64_t)nt * Tile::TN;
    floatx16 acc[Tile::FM][Tile::FN];
    Tile::template run<RAGGED>(At, K, Wt, N, rows_valid, cols_valid, K, stages, acc);

    const int64_t obase = ((int64_t)c * Mc + (int64_t)mt * Tile::TM) * N + (int64_t)nt * Tile::TN;
    store_tile<Tile, ODT, RAGGED, kPolicyPlain, false>(
        reinterpret_cast<char*>(a.out) + obase * (ODT == kBF16 ? 2 : 4), N, rows_valid, cols_valid,
        acc, stages);
  }

  // the last workgroup out leaves the workspace zeroed
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      for (int w = 0; w < P + 4; ++w)
        __hip_atomic_store(&ws[w], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <class Tile, bool RAGGED, int ODT>
static int launch_k(const AgGemmArgs& a, hipStream_t s) {
  auto kern = &ag_gemm_kernel<Tile, RAGGED, ODT>;
  int grid = 0;
  hipError_t e = persistent_grid(reinterpret_cast<const void*>(kern), Tile::NT,
                                 (int64_t)a.P * a.mtiles * a.ntiles, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Tile::NT), 0, s, a);
  return hipGetLastError();
}

// full tiles take the direct-to-LDS mainloop, ragged ones the register-staged one
template <int TM, int TN, int ODT>
static int launch_tile(const AgGemmArgs& a, hipStream_t s) {
  using Staged = TileBf16<TM, TN, 2, 2>;
  using Direct = TileBf16Direct<TM, TN, 2, 2>;
  // the direct tile takes full tiles whose operands it can address with 32-bit offsets
  const bool ragged = (a.Mc % TM) || (a.N % TN) || !Direct::k_fits(a.K) ||
                      !Direct::operands_fit(a.K, a.N, a.K);
  return ragged ? launch_k<Staged, true, ODT>(a, s) : launch_k<Direct, false, ODT>(a, s);
}

template <int TM, int TN>
static int launch_out(const AgGemmArgs& a, hipStream_t s) {
  return a.out_dt == kBF16 ? launch_tile<TM, TN, kBF16>(a, s) : launch_tile<TM, TN, kF32>(a, s);
}

int launch_ag_gemm(const AgGemmArgs& a, int tm, int tn, hipStream_t s) {
  if (tm == 256 && tn == 256) return launch_out<256, 256>(a, s);
  if (tm == 128 && tn == 128) return launch_out<128, 128>(a, s);
  return kNoKernel;
}

}  // namespace hocf
