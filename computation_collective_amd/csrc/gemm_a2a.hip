// GEMM + All-to-All (the mixture-of-experts combine), fused in one kernel.
//
// SC24 ("Optimizing Distributed ML Communication with Fused
// Computation-Collective Operations", abstract) names GEMM + All-to-All, for
// MoE layers, among its three fused prototypes: the expert GEMM's result
// rows go back to the ranks their tokens came from as soon as a workgroup
// has computed them, while other workgroups still compute.
//
// This rank holds E experts.  The token rows it received are grouped by
// expert, each group padded to whole tiles of tile_m rows (the block-aligned
// layout of a grouped GEMM; padding rows carry dest = -1).  Work item = one
// tile_m x 256 tile (expert e, row tile, column tile) of Y_e = X_e . W_e
// (tile_m = 256 or 128), computed with
// the direct-to-LDS MFMA mainloop; items are dealt statically (every tile
// costs the same).  The epilogue scatters the tile's rows: row i goes to
// window dest[i], row slot[i] -- a data-dependent destination per row, so
// each wave stages a 32-row block in LDS and stores it with per-lane 8-byte
// device-coherent stores, each store instruction covering whole 128-byte
// lines of one or two destination rows.  The workgroup counts the rows it
// delivered per destination (in LDS), waits for its stores, and adds the
// counts to one arrival counter per destination; the workgroup whose add
// completes a destination's expected count (its send count x column tiles)
// stores the epoch into that window's flag.  A destination that receives
// nothing gets its flag from the last workgroup to finish.  Rows naming a
// destination or slot out of range are skipped and reported
// (HOCF_ERR_BAD_INDEX); their destination's flag is then never set.
#include "internal.hpp"
#include "mfma_tile.hpp"
#include "publish.hpp"
#include "sync.hpp"

namespace hocf {

// The tile's rows -> their destination windows.  Begins with a barrier (the
// mainloop's last LDS reads are done) and uses the stage arrays for staging;
// s_route[r] holds tile row r's (dest, slot), loaded before the mainloop, and
// s_win the P window bases (so that the store loop waits on nothing but LDS:
// a per-lane read of the kernel's argument array would be a global load, and
// its wait would also wait for every store issued before it).
template <class Tile, int ODT>
__device__ __forceinline__ void scatter_rows(const GemmA2aArgs& a, int col0,
                                             const floatx16 (&acc)[Tile::FM][Tile::FN],
                                             char* const (&stages)[4], const int2* s_route, const uint64_t* s_win,
                                             uint32_t* s_cnt) {
  using L = PublishLayout<Tile, ODT>;
  constexpr int PPR = L::RB / 8;   // 8-byte pieces per staged row
  constexpr int RPI = 64 / PPR;    // rows per store instruction
  constexpr int NIT = 32 / RPI;    // store instructions per 32-row block
  static_assert(64 % PPR == 0 && RPI >= 1, "scatter layout");
  const int wave = threadIdx.x >> 6;
  const int lane = opaque_lane();
  const int wm = wave / Tile::WN, wn = wave % Tile::WN;
  const int lr = lane & 31, half = lane >> 5;
  const int sr = lane / PPR, pc = lane % PPR;  // staged row (within an instruction) and piece
  const int tcol = col0 + wn * Tile::WTN + pc * (8 / L::ES);  // first output column of this lane
  __syncthreads();
  char* area = L::area(stages, wave);
#pragma unroll
  for (int i = 0; i < Tile::FM; ++i) {
    // accumulator block row i -> staging rows 0..31 (row lr of this lane)
#pragma unroll
    for (int j = 0; j < Tile::FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * j + 8 * g + 4 * half;  // wave-local column
        const int byte = col * L::ES;
        char* p = area + L::at(lr, byte >> 4) + (byte & 15);
        if constexpr (ODT == kBF16) {
          *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                                               pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
        } else {
          *reinterpret_cast<floatx4*>(p) =
              floatx4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
      }
    // staged rows -> their destinations; LDS operations of one wave complete
    // in order, so no barrier is needed between the staging and the reads
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + sr;  // staged row
      const u32x2 v = *reinterpret_cast<const u32x2*>(area + L::at(r, pc >> 1) + (pc & 1) * 8);
      const int2 route = s_route[wm * Tile::WTM + 32 * i + r];
      const int d = route.x, s = route.y;
      if (d < 0) continue;  // padding row
      if (d >= a.P || s < 0 || s >= a.cap) {
        if (pc == 0) report_status(a.sync, kErrBadIndex);
        continue;
      }
      // a global (not flat) address: a flat store would also count against the LDS counter
      typedef __attribute__((address_space(1))) uint64_t gu64;
      gu64* p = (gu64*)(s_win[d] + (uint64_t)(((int64_t)s * a.N + tcol) * L::ES));
      // relaxed device-scope store: written through to the memory side (no L2-wide fence needed)
      __hip_atomic_store(p, __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (pc == 0 && wn == 0) atomicAdd(&s_cnt[d], 1u);  // one piece per row and column tile
    }
  }
}

// One tile of the grouped GEMM (whole, or one of its half- or
// quarter-height parts, with the tile shape T), scattered; returns after the
// barrier that follows its stores.
template <class T, int ODT>
__device__ __forceinline__ void a2a_tile(const GemmA2aArgs& a, int64_t row0, int e, int nt,
                                         char* const (&stages)[4], int2* s_route, const uint64_t* s_win,
                                         uint32_t* s_cnt) {
  const int tid = threadIdx.x;
  const uint16_t* At = a.X + row0 * a.K;
  const uint16_t* Wt = a.W + (int64_t)e * a.K * a.N + (int64_t)nt * T::TN;
  // the rows' routes, loaded now so that their latency hides behind the mainloop
  int2 route = {-1, -1};
  if (tid < T::TM) route = int2{a.dest[row0 + tid], a.slot[row0 + tid]};
  floatx16 acc[T::FM][T::FN];
  T::template run<false>(At, a.K, Wt, a.N, T::TM, T::TN, a.K, stages, acc);
  // (the previous tile's scatter read s_route before the barrier that ended it)
  if (tid < T::TM) s_route[tid] = route;
  scatter_rows<T, ODT>(a, nt * T::TN, acc, stages, s_route, s_win, s_cnt);
  wait_memory();  // this thread's row stores have completed
  __syncthreads();
}

template <class Tile, int ODT>
__global__ __launch_bounds__(Tile::NT) void gemm_a2a_kernel(GemmA2aArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem0[Tile::SMEM_BYTES];
  __shared__ __attribute__((aligned(1024))) char smem1[Tile::NST > 1 ? Tile::SMEM_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char smem2[Tile::NST > 2 ? Tile::SMEM_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char smem3[Tile::NST > 3 ? Tile::SMEM_BYTES : 16];
  char* const stages[4] = {smem0, smem1, smem2, smem3};
  __shared__ uint32_t s_cnt[kMaxP];
  __shared__ int2 s_route[Tile::TM];  // (dest, slot) of the current tile's rows
  __shared__ uint64_t s_win[kMaxP];    // window bases
  __shared__ int s_last;
  static_assert(Tile::NT >= Tile::TM, "one thread per tile row loads its route");

  const int tid = threadIdx.x;
  uint32_t* arrived = a.ws + kWsExtra;  // [P] pieces delivered per destination
  if (tid < kMaxP) s_cnt[tid] = 0;
  if (tid < a.P) s_win[tid] = reinterpret_cast<uint64_t>(a.win_data[tid]);  // (read after the scatter's barrier)

  // round k of the static schedule: the workgroups of one XCD take a
  // contiguous run of items, and within an expert the items run in blocks of
  // (up to) 8 column tiles, row tile by row tile, so such a run covers a few
  // row tiles by 8 column tiles, sharing their X and W panels in that XCD's L2
  constexpr int kColBlock = 8;
  //
  // Tiles [keep, total) -- the last, partial round of whole tiles -- run as
  // `split` (2 or 4) tiles of 256 / split rows each, so that round takes a
  // half or a quarter as long (the same rows, each computed once; only
  // 256-row tiles with bf16 output split).
  constexpr bool kSplits = ODT == kBF16 && Tile::TM == 256;
  using Half = TileBf16Direct<kSplits ? Tile::TM / 2 : Tile::TM, Tile::TN, 2, 2>;
  using Quarter = TileBf16Direct<kSplits ? Tile::TM / 4 : Tile::TM, Tile::TN, 2, 2>;
  static_assert(!kSplits || (Half::SMEM_BYTES <= Tile::SMEM_BYTES && Half::NT == Tile::NT &&
                             Quarter::SMEM_BYTES <= Tile::SMEM_BYTES && Quarter::NT == Tile::NT),
                "part tiles");
  const int split = kSplits ? a.split : 1;
  const int nwork = a.keep + split * (a.total - a.keep);
  const int first = (int)xcd_contiguous(blockIdx.x, gridDim.x);
  for (int w = first; w < nwork; w += gridDim.x) {
    const bool part = w >= a.keep;
    const int item = part ? a.keep + (w - a.keep) / split : w;
    int e = 0;
    while (e + 1 < a.E && item >= a.tile_off[e + 1]) ++e;
    const int local = item - a.tile_off[e];
    const int mtiles = (a.tile_off[e + 1] - a.tile_off[e]) / a.ntiles;
    const int nb = local / (mtiles * kColBlock);               // column block
    const int width = min(kColBlock, a.ntiles - nb * kColBlock);
    const int j = local - nb * mtiles * kColBlock;
    const int mt = j / width, nt = nb * kColBlock + j % width;
    const int64_t row0 = a.row_off[e] + (int64_t)mt * Tile::TM;
    if constexpr (kSplits) {
      if (part && split == 4)
        a2a_tile<Quarter, ODT>(a, row0 + (int64_t)((w - a.keep) % 4) * Quarter::TM, e, nt, stages, s_route, s_win,
                               s_cnt);
      else if (part)
        a2a_tile<Half, ODT>(a, row0 + (int64_t)((w - a.keep) % 2) * Half::TM, e, nt, stages, s_route, s_win, s_cnt);
      else
        a2a_tile<Tile, ODT>(a, row0, e, nt, stages, s_route, s_win, s_cnt);
    } else {
      a2a_tile<Tile, ODT>(a, row0, e, nt, stages, s_route, s_win, s_cnt);
    }
    if (tid < a.P) {
      const uint32_t c = s_cnt[tid];
      s_cnt[tid] = 0;  // (the next tile's counts start after the next scatter's first barrier)
      if (c) {
        const uint32_t prev = __hip_atomic_fetch_add(&arrived[tid], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev + c == a.expected[tid]) {
          // every row this rank sends to destination tid is in its window
          __hip_atomic_store(&arrived[tid], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&a.win_flags[tid][0], a.sync.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  // the last workgroup out flags the destinations that receive no rows, and
  // clears every arrival counter: a destination whose rows were not all
  // delivered (a row skipped for a bad destination or slot) never reached
  // its expected count, so its counter still holds what did arrive
  if (finish_workgroup_last(a.ws, &s_last)) {
    if (tid < a.P && a.expected[tid] == 0)
      __hip_atomic_store(&a.win_flags[tid][0], a.sync.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < a.P) __hip_atomic_store(&arrived[tid], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <class Tile, int ODT>
static int launch_k(const GemmA2aArgs& a0, hipStream_t s) {
  auto kern = &gemm_a2a_kernel<Tile, ODT>;
  constexpr bool kSplits = ODT == kBF16 && Tile::TM == 256;  // (as in the kernel)
  int grid = 0;
  hipError_t e = persistent_grid(reinterpret_cast<const void*>(kern), Tile::NT,
                                 kSplits ? 4 * (int64_t)a0.total : a0.total, &grid);
  if (e != hipSuccess) return e;
  // split the last, partial round of whole tiles into quarter- or
  // half-height tiles, the finest whose parts still fit in one round of the
  // grid (the kernel splits only 256-row tiles with bf16 output)
  GemmA2aArgs a = a0;
  const int rem = a.total % grid;
  a.split = !kSplits || rem == 0 ? 1 : 4 * rem <= grid ? 4 : 2 * rem <= grid ? 2 : 1;
  a.keep = a.split > 1 ? a.total - rem : a.total;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Tile::NT), 0, s, a);
  return hipGetLastError();
}

template <class Tile>
static int launch_tile(const GemmA2aArgs& a, hipStream_t s) {
  return a.out_dt == kBF16 ? launch_k<Tile, kBF16>(a, s) : launch_k<Tile, kF32>(a, s);
}

int launch_gemm_a2a(const GemmA2aArgs& a, int tile_m, hipStream_t s) {
  if (tile_m == 256) return launch_tile<TileBf16Direct<256, 256, 2, 2>>(a, s);
  // (128-row tiles: bf16 output only -- an fp32 staging row block does not fit their stage arrays)
  if (tile_m == 128 && a.out_dt == kBF16) return launch_k<TileBf16Direct<128, 256, 2, 2>, kBF16>(a, s);
  return kNoKernel;
}

}  // namespace hocf
