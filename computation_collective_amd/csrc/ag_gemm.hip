// AllGather + GEMM with chunk-gated tile claiming.
//
// mKernel news item ("GPU-vezérelt kommunikációval gyorsítják az
// AI-betanítást a kutatók"): AllGather + GEMM is one of its five fused
// kernels, overlapping the arriving chunks with compute at tile/chunk
// granularity inside one persistent kernel.
//
// Chunk c of the gathered A (rows [c*Mc, (c+1)*Mc)) is written by someone
// else -- a copy engine, another stream, a peer -- which then sets
// chunk_flags[c] = epoch.  The kernel's persistent workgroups claim output
// tiles only from chunks whose flag has arrived, earliest arrival first:
// the first workgroup that sees a chunk's flag appends the chunk to an
// arrival list in the workspace, and every workgroup walks that list in
// order, taking the next unclaimed tile of the first chunk that still has
// one.  A workgroup acquires (system scope: the writer may be a DMA engine)
// the first time it uses a chunk.  Tiles are computed identically whatever
// the order, so the output does not depend on the release order.
//
// Every wait is bounded: after the time limit (or an abort request) the
// waiting workgroup records the error and exits, so the kernel always ends.
//
// Workspace words after the common queue block (kWsExtra):
//   [0, P)      per-chunk tile counters
//   P           mask of chunks already appended to the arrival list
//   P + 1       arrival list length
//   [P+2, 2P+2) arrival list (chunk id + 1)
//   2P + 2      count of finished workgroups (the last one resets all words)
#include "internal.hpp"
#include "mfma_tile.hpp"
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

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.P, N = a.N, K = a.K, Mc = a.Mc;
  const int tpc = a.mtiles * a.ntiles;
  uint32_t* ws = a.ws + kWsExtra;
  uint32_t* cnt = ws;
  uint32_t* reg_mask = ws + P;
  uint32_t* arr_len = ws + P + 1;
  uint32_t* arr = ws + P + 2;
  uint32_t* done = ws + 2 * P + 2;
  const uint32_t all = (P >= 32) ? 0xffffffffu : ((1u << P) - 1u);

  // thread 0's private state
  uint32_t seen = 0;       // chunks whose flag this workgroup has acquired
  uint32_t exhausted = 0;  // chunks with no tile left
  Deadline dl{now_ticks(), a.sync.timeout_ticks};

  for (;;) {
    __syncthreads();  // keeps the thread-0 claim region apart from the previous iteration
    if (tid == 0) {
      int chunk = -1, tile = -1;
      for (;;) {
        // 1. look for newly arrived chunks and append them to the arrival list
        for (int c = 0; c < P; ++c) {
          if (seen & (1u << c)) continue;
          if (load_flag_system(&a.chunk_flags[c]) == a.sync.epoch) {
            acquire_system();
            seen |= 1u << c;
            const uint32_t old = __hip_atomic_fetch_or(reg_mask, 1u << c, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            if (!(old & (1u << c))) {
              const uint32_t pos = __hip_atomic_fetch_add(arr_len, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(&arr[pos], (uint32_t)c + 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
        // 2. take a tile from the earliest-arrived chunk that has one
        const uint32_t len = __hip_atomic_load(arr_len, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (uint32_t i = 0; i < len && i < (uint32_t)P; ++i) {
          const uint32_t e = __hip_atomic_load(&arr[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (e == 0) break;  // slot claimed but not yet written
          const int c = (int)e - 1;
          if ((exhausted | ~seen) & (1u << c)) continue;  // only chunks this WG acquired
          const uint32_t t = __hip_atomic_fetch_add(&cnt[c], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
          if ((int)t < tpc) { chunk = c; tile = (int)t; break; }
          exhausted |= 1u << c;
        }
        if (chunk >= 0) { dl.start = now_ticks(); break; }  // the bound is per wait
        if (exhausted == all) break;
        // 3. nothing to do yet: bounded wait
        if (a.sync.abort_flag && load_flag_system(a.sync.abort_flag) != 0u) {
          report_status(a.sync, kErrAborted);
          break;
        }
        if (dl.expired()) {
          report_status(a.sync, kErrTimeout);
          break;
        }
        __builtin_amdgcn_s_sleep(8);
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
    Tile::template store_acc<ODT, RAGGED>(
        reinterpret_cast<char*>(a.out) + obase * (ODT == kBF16 ? 2 : 4), N, rows_valid, cols_valid,
        acc);
  }

  // the last workgroup out leaves the workspace zeroed
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      for (int w = 0; w < 2 * P + 3; ++w)
        __hip_atomic_store(&ws[w], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <class Tile, bool RAGGED, int ODT>
static hipError_t launch_k(const AgGemmArgs& a, hipStream_t s) {
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
static hipError_t launch_tile(const AgGemmArgs& a, hipStream_t s) {
  using Staged = TileBf16<TM, TN, 2, 2>;
  using Direct = TileBf16Direct<TM, TN, 2, 2>;
  const bool ragged = (a.Mc % TM) || (a.N % TN) || (a.K % Direct::KSTEP);
  return ragged ? launch_k<Staged, true, ODT>(a, s) : launch_k<Direct, false, ODT>(a, s);
}

template <int TM, int TN>
static hipError_t launch_out(const AgGemmArgs& a, hipStream_t s) {
  return a.out_dt == kBF16 ? launch_tile<TM, TN, kBF16>(a, s) : launch_tile<TM, TN, kF32>(a, s);
}

hipError_t launch_ag_gemm(const AgGemmArgs& a, int tm, int tn, hipStream_t s) {
  if (tm == 256 && tn == 256) return launch_out<256, 256>(a, s);
  if (tm == 128 && tn == 128) return launch_out<128, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace hocf
