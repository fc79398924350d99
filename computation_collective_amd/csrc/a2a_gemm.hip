// All-to-All + GEMM (the mixture-of-experts dispatch followed by the expert
// GEMM), fused: expert tiles start as soon as the token rows they need have
// landed, while other workgroups are still delivering rows.
//
// The mKernel news item ("GPU-vezérelt kommunikációval gyorsítják az
// AI-betanítást a kutatók", section on its five fused kernels) lists MoE
// Dispatch + GEMM; SC24 ("Optimizing Distributed ML Communication with Fused
// Computation-Collective Operations", abstract) fuses collectives with their
// computations at workgroup granularity.  One rank's share: P source ranks
// hold B tokens each with their top-k router choices; this rank owns experts
// e0 .. e0+E-1.  The All-to-All delivers, for each local expert, the token
// rows of the (source, token, choice) pairs that picked it, in that order,
// each expert's group padded with zero rows to whole tiles (the
// block-aligned layout of a grouped GEMM); then Y = recv . W_e per group.
//
// Three kernels on the caller's stream:
//   1. count: one workgroup per chunk of kA2gChunk router entries of one
//      source: a histogram of the chunk's local experts, and of its pairs
//      landing here at all;
//   2. scan (one workgroup): exclusive scans of every histogram column over
//      the chunks -- each chunk's first row inside each expert group, and
//      its first slot among its source's pairs (the per-source column
//      restarts at every source) -- then the padded group offsets, the
//      expert tiles, the send counts, and zeroed arrival counters;
//   3. the fused kernel (persistent): a workgroup first claims delivery
//      items from one counter -- the padding fills (each group's padding in
//      a few pieces), then the chunks -- and, once that counter is
//      exhausted, expert tiles from eight queues, one per XCD, each a
//      contiguous run of the tile list (expert, row tile, column tile), so
//      an XCD's tiles share row tiles and W panels in its L2.  A chunk item
//      ranks the chunk's pairs per expert with wave ballots, copies their
//      token rows into the receive buffer with device-coherent stores,
//      writes dest and slot, then counts the rows landed per row tile.  A
//      tile waits (bounded) until its row tile has all its rows, then runs
//      the direct-to-LDS MFMA mainloop of the other GEMMs and stores Y; so
//      the tiles whose rows land first start while other workgroups still
//      deliver.  A tile is claimed only after every delivery item has been
//      claimed by a running workgroup (which waits on nothing), so the
//      kernel needs no co-residency to finish.
// The unfused baseline runs the scatter items as one kernel and the tiles as
// the next (bit-identical results).
#include "internal.hpp"
#include "mfma_tile.hpp"
#include "publish.hpp"
#include "sync.hpp"

namespace hocf {

// Each expert group's padding (up to tile_m - 1 rows) is filled in this
// many pieces, so that no single workgroup writes all of it.
constexpr int kA2gPadPieces = 8;

// 1. Histogram of one chunk: hist[c][e] for local expert e, hist[c][E] for
// all of the chunk's pairs that land on this rank.
__global__ __launch_bounds__(kA2gChunk) void a2g_count_kernel(A2aGemmArgs a) {
  __shared__ uint32_t h[kMaxExperts + 1];
  const int tid = threadIdx.x, c = blockIdx.x, E = a.E;
  if (tid <= E) h[tid] = 0;
  __syncthreads();
  const int p = c / a.cps, piece = c % a.cps;
  const int64_t per = (int64_t)a.B * a.topk;
  const int64_t i = (int64_t)piece * kA2gChunk + tid;
  if (i < per) {
    const int64_t le = (int64_t)a.experts[(int64_t)p * per + i] - a.e0;
    if (le >= 0 && le < E) {
      atomicAdd(&h[le], 1u);
      atomicAdd(&h[E], 1u);
    }
  }
  __syncthreads();
  if (tid <= E) a.hist[(int64_t)c * (E + 1) + tid] = h[tid];
}

// 2. Scans, group offsets, send counts (one workgroup of 256 threads).
__global__ __launch_bounds__(256) void a2g_scan_kernel(A2aGemmArgs a) {
  __shared__ uint32_t tot[kMaxExperts + 1];
  __shared__ uint32_t src0[kMaxP + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, C = a.C, W1 = E + 1;
  // every column: base[c][i] = sum over chunks c' < c of hist[c'][i]; one
  // wave per column, each lane a contiguous run of chunks
  const int run = (C + 63) / 64;
  for (int i = wave; i <= E; i += 4) {
    const int c0 = min(C, lane * run), c1 = min(C, c0 + run);
    uint32_t s = 0;
    for (int c = c0; c < c1; ++c) s += a.hist[(int64_t)c * W1 + i];
    uint32_t incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    uint32_t r = incl - s;
    for (int c = c0; c < c1; ++c) {
      const uint32_t h = a.hist[(int64_t)c * W1 + i];
      a.base[(int64_t)c * W1 + i] = r;
      r += h;
    }
    if (lane == 63) tot[i] = incl;
  }
  __syncthreads();
  // the last column restarts at every source: a chunk's first slot is its
  // count minus its source's first chunk's; a source's pairs here are its
  // send count
  if (tid < a.P) src0[tid] = a.base[(int64_t)tid * a.cps * W1 + E];
  if (tid == 0) src0[a.P] = tot[E];
  __syncthreads();
  for (int c = tid; c < C; c += 256) a.base[(int64_t)c * W1 + E] -= src0[c / a.cps];
  if (tid < a.P) a.send_counts[tid] = (int64_t)(src0[tid + 1] - src0[tid]);
  if (tid == 0) {
    uint32_t row = 0, tile = 0;
    for (int e = 0; e < E; ++e) {
      const uint32_t n = tot[e];
      const uint32_t padded = (n + a.tile_m - 1) / a.tile_m * a.tile_m;
      a.grp[e] = row;
      a.cnt[e] = n;
      a.toff[e] = tile;
      a.expert_offsets[e] = row;
      row += padded;
      tile += padded / a.tile_m * a.ntiles;
    }
    a.grp[E] = row;
    a.toff[E] = tile;
    a.expert_offsets[E] = row;
    const bool over = (int64_t)row > a.cap;
    a.misc[0] = 0;
    a.misc[1] = over ? 1u : 0u;
    a.misc[2] = over ? 0u : tile;
    for (int q = 0; q < kNumQueues; ++q) a.misc[4 + q] = 0;
    if (over) report_status(a.sync, kErrCapacity);
  }
  for (int i = tid; i < a.nrt; i += 256) a.arrivals[i] = 0;
}

// Copies (or, with src == nullptr, zeroes) one row of K bf16 elements into
// the receive buffer with device-coherent 16-byte stores; called by one wave.
// Loads are unconditional (pieces past the row's end re-read its last piece,
// never stored): a load under a per-lane condition becomes a branch with a
// full wait, which would serialise them.
__device__ __forceinline__ void move_row(const uint16_t* src, uint16_t* dst, int K, int lane) {
  const __amdgpu_buffer_rsrc_t rd = raw_rsrc(dst);
  constexpr int U = 8;  // 16-byte pieces per lane in flight
  for (int k0 = lane * 8; k0 < K; k0 += 64 * 8 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = src ? *reinterpret_cast<const u32x4*>(src + min(k0 + u * 512, K - 8)) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * 512;
      if (k < K) st_dev16(rd, (uint32_t)k * 2, 0, v[u]);
    }
  }
}

// Copies R token rows at once (all their loads issued before any store), so a
// wave keeps R rows' worth of loads in flight; called by one wave.  src[r] and
// dst[r] are wave-uniform.
template <int R>
__device__ __forceinline__ void move_rows(const uint16_t* const (&src)[R], uint16_t* const (&dst)[R], int K,
                                          int lane) {
  constexpr int U = 8;
  for (int k0 = lane * 8; k0 < K; k0 += 64 * 8 * U) {
    u32x4 v[R][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(k0 + u * 512, K - 8);
#pragma unroll
      for (int r = 0; r < R; ++r) v[r][u] = *reinterpret_cast<const u32x4*>(src[r] + k);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * 512;
      if (k < K) {
#pragma unroll
        for (int r = 0; r < R; ++r) st_dev16(raw_rsrc(dst[r]), (uint32_t)k * 2, 0, v[r][u]);
      }
    }
  }
}

// Piece `piece` (of kA2gPadPieces) of the padding rows of expert e's group:
// zero token rows, dest = slot = -1; they all lie in the group's last row
// tile.
template <int NT>
__device__ __forceinline__ void a2g_pad(const A2aGemmArgs& a, int e, int piece) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t pad0 = a.grp[e] + a.cnt[e], pad1 = a.grp[e + 1];
  const uint32_t per = (pad1 - pad0 + kA2gPadPieces - 1) / kA2gPadPieces;
  const uint32_t r0 = min(pad1, pad0 + per * (uint32_t)piece), r1 = min(pad1, r0 + per);
  for (uint32_t r = r0 + (uint32_t)wave; r < r1; r += NT / 64)
    move_row(nullptr, a.recv + (int64_t)r * a.K, a.K, lane);
  for (uint32_t r = r0 + (uint32_t)tid; r < r1; r += NT) {
    a.dest[r] = -1;
    a.slot[r] = -1;
  }
  wait_memory();
  __syncthreads();
  if (tid == 0 && r1 > r0)
    __hip_atomic_fetch_add(&a.arrivals[(r1 - 1) / a.tile_m], r1 - r0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Chunk c: rank its pairs, deliver their token rows, count them in.
// `scratch` is LDS the caller does not use meanwhile (>= 2 KB + 256 ints).
template <int NT>
__device__ __forceinline__ void a2g_chunk(const A2aGemmArgs& a, int c, char* scratch) {
  static_assert(NT >= kA2gChunk, "one thread per router entry");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, W1 = E + 1;
  uint32_t* cw = reinterpret_cast<uint32_t*>(scratch);                  // [NT/64][E+1] counts per wave
  int2* pairs = reinterpret_cast<int2*>(scratch + (NT / 64) * (kMaxExperts + 1) * 4);  // [kA2gChunk]: (row, token)
  const int p = c / a.cps, piece = c % a.cps;
  const int64_t per = (int64_t)a.B * a.topk;
  const int64_t i = (int64_t)piece * kA2gChunk + tid;
  int le = -1;
  if (tid < kA2gChunk && i < per) {
    const int64_t v = (int64_t)a.experts[(int64_t)p * per + i] - a.e0;
    if (v >= 0 && v < E) le = (int)v;
  }
  // ranks within the chunk, in entry order: per expert, and among all pairs landing here
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t rank_e = 0, rank_l = 0;
  for (int e = 0; e < E; ++e) {
    const uint64_t m = __ballot(le == e);
    if (le == e) rank_e = (uint32_t)__popcll(m & below);
    if (lane == 0) cw[wave * W1 + e] = (uint32_t)__popcll(m);
  }
  const uint64_t ml = __ballot(le >= 0);
  if (le >= 0) rank_l = (uint32_t)__popcll(ml & below);
  if (lane == 0) cw[wave * W1 + E] = (uint32_t)__popcll(ml);
  __syncthreads();
  int row = -1;
  if (le >= 0) {
    for (int w = 0; w < wave; ++w) {
      rank_e += cw[w * W1 + le];
      rank_l += cw[w * W1 + E];
    }
    const int64_t cb = (int64_t)c * W1;
    row = (int)(a.grp[le] + a.base[cb + le] + rank_e);
    a.dest[row] = p;
    a.slot[row] = (int32_t)(a.base[cb + E] + rank_l);
  }
  // the chunk's pairs in entry order (their rank among the pairs landing
  // here), each with its row and its token; then one wave per two pairs
  if (row >= 0) pairs[rank_l] = int2{row, (int)(((int64_t)piece * kA2gChunk + tid) / a.topk)};
  uint32_t n_loc = 0;
  for (int w = 0; w < NT / 64; ++w) n_loc += cw[w * W1 + E];
  __syncthreads();
  constexpr int RW = 4;  // rows a wave moves at once
  for (uint32_t k = RW * (uint32_t)wave; k < n_loc; k += RW * (NT / 64)) {
    if (k + RW <= n_loc) {
      const uint16_t* sr[RW];
      uint16_t* dr[RW];
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const int2 q = pairs[k + r];
        const int rr = __builtin_amdgcn_readfirstlane(q.x), bb = __builtin_amdgcn_readfirstlane(q.y);
        sr[r] = a.X + ((int64_t)p * a.B + bb) * a.K;
        dr[r] = a.recv + (int64_t)rr * a.K;
      }
      move_rows<RW>(sr, dr, a.K, lane);
    } else {
      for (uint32_t kk = k; kk < n_loc; ++kk) {
        const int2 q = pairs[kk];
        const int rr = __builtin_amdgcn_readfirstlane(q.x), bb = __builtin_amdgcn_readfirstlane(q.y);
        move_row(a.X + ((int64_t)p * a.B + bb) * a.K, a.recv + (int64_t)rr * a.K, a.K, lane);
      }
    }
  }
  wait_memory();  // this thread's row stores have completed
  __syncthreads();
  // count the rows in: the chunk's rows of expert e are one contiguous run
  // (first = its group's start + the chunk's scan value), so thread e adds
  // one count per row tile the run touches (a few atomics per chunk, not one
  // per row)
  if (tid < E) {
    uint32_t n = 0;
    for (int w = 0; w < NT / 64; ++w) n += cw[w * W1 + tid];
    if (n > 0) {
      const uint32_t tm = (uint32_t)a.tile_m;
      const uint32_t first = a.grp[tid] + a.base[(int64_t)c * W1 + tid], last = first + n - 1;
      for (uint32_t rt = first / tm; rt <= last / tm; ++rt) {
        const uint32_t lo = max(first, rt * tm), hi = min(last, rt * tm + tm - 1);
        __hip_atomic_fetch_add(&a.arrivals[rt], hi - lo + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// 3. The fused kernel (SCATTER and GEMM), or one half of the unfused pair.
template <class Tile, int ODT, bool SCATTER, bool GEMM>
__global__ __launch_bounds__(Tile::NT) void a2a_gemm_kernel(A2aGemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem0[Tile::SMEM_BYTES];
  __shared__ __attribute__((aligned(1024))) char smem1[Tile::NST > 1 ? Tile::SMEM_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char smem2[Tile::NST > 2 ? Tile::SMEM_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char smem3[Tile::NST > 3 ? Tile::SMEM_BYTES : 16];
  char* const stages[4] = {smem0, smem1, smem2, smem3};
  __shared__ int64_t s_item;
  __shared__ int s_ok;
  static_assert(Tile::SMEM_BYTES >= (Tile::NT / 64) * (kMaxExperts + 1) * 4 + kA2gChunk * 8, "chunk scratch");
  constexpr bool FUSED = SCATTER && GEMM;
  const int tid = threadIdx.x;
  if (a.misc[1] != 0) return;  // more rows than the receive buffer holds: nothing is delivered
  const int E = a.E;
  const int64_t npad = (int64_t)E * kA2gPadPieces;
  const int64_t nscatter = SCATTER ? npad + a.C : 0;
  // Delivery items (the padding pieces, then the chunks) are dealt in order
  // by one counter; tiles by eight queues, one per XCD (home queue blockIdx
  // mod 8, then the others), each a contiguous run of the tile list
  // (expert, row tile, column tile), so an XCD's tiles share row tiles and
  // W panels in its L2.  Fused, a workgroup turns to the tile queues once
  // the delivery counter is exhausted: every tile then waits only on items
  // already claimed.  Item numbers: delivery items [0, nscatter), tile t is
  // nscatter + t.
  const uint32_t ntile = GEMM ? a.misc[2] : 0u;
  bool delivering = SCATTER;  // (thread 0) the delivery counter may have items left
  uint32_t* tq = &a.misc[4];
  auto qbeg = [&](int q) { return (uint32_t)(((uint64_t)ntile * q) / kNumQueues); };
  int qoff = 0;
  if constexpr (GEMM) {
    // received rows went to memory with device-coherent stores and none is
    // read before it has landed, so one invalidate of this XCD's L2 here (lines
    // older than this call) lets the tiles read them with ordinary loads
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }

  for (;;) {
    __syncthreads();  // the previous item's LDS use is over
    if (tid == 0) {
      int64_t it = -1;
      if (delivering) {
        const uint32_t v = __hip_atomic_fetch_add(&a.misc[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int64_t)v < nscatter) it = v;
        else delivering = false;
      }
      if (it < 0 && GEMM) {
        const int home = (int)(blockIdx.x % kNumQueues);
        while (qoff < kNumQueues) {
          const int q = (home + qoff) % kNumQueues;
          const uint32_t v = __hip_atomic_fetch_add(&tq[q], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (v < qbeg(q + 1) - qbeg(q)) { it = nscatter + qbeg(q) + v; break; }
          ++qoff;
        }
      }
      s_item = it;
    }
    __syncthreads();
    const int64_t item = uniform64(s_item);
    if (item < 0) break;
    if (SCATTER && item < npad) {
      a2g_pad<Tile::NT>(a, (int)(item / kA2gPadPieces), (int)(item % kA2gPadPieces));
      continue;
    }
    if (SCATTER && item < nscatter) {
      a2g_chunk<Tile::NT>(a, (int)(item - npad), smem0);
      continue;
    }
    // an expert tile of the list: (expert e, row tile mt, column tile nt)
    const uint32_t t = (uint32_t)(item - nscatter);
    int e = 0;
    while (e + 1 < E && t >= a.toff[e + 1]) ++e;
    const uint32_t local = t - a.toff[e];
    const int mt = (int)(local / (uint32_t)a.ntiles), nt = (int)(local % (uint32_t)a.ntiles);
    const uint32_t row0 = a.grp[e] + (uint32_t)mt * Tile::TM;
    if constexpr (FUSED) {
      // the row tile's rows (copied or zero-filled by items claimed earlier)
      if (tid == 0) {
        const uint32_t* cnt = &a.arrivals[row0 / Tile::TM];
        const Deadline dl{now_ticks(), a.sync.timeout_ticks};
        int w = kWaitOk;
        while (load_flag_agent(cnt) < (uint32_t)Tile::TM) {
          if (abort_requested(a.sync)) { w = kWaitAborted; break; }
          if (dl.expired()) { w = kWaitTimeout; break; }
          __builtin_amdgcn_s_sleep(16);  // (about a microsecond: waiting tiles poll lightly while rows move)
        }
        report_wait(a.sync, w);
        s_ok = w == kWaitOk;
      }
      __syncthreads();
      if (!uniform(s_ok)) break;
    }
    const uint16_t* At = a.recv + (int64_t)row0 * a.K;
    const uint16_t* Wt = a.W + (int64_t)e * a.K * a.N + (int64_t)nt * Tile::TN;
    floatx16 acc[Tile::FM][Tile::FN];
    Tile::template run<false>(At, a.K, Wt, a.N, Tile::TM, Tile::TN, a.K, stages, acc);
    const int64_t obase = (int64_t)row0 * a.N + (int64_t)nt * Tile::TN;
    store_tile<Tile, ODT, false, kPolicyPlain, false>(
        reinterpret_cast<char*>(a.Y) + obase * (ODT == kBF16 ? 2 : 4), a.N, Tile::TM, Tile::TN, acc, stages);
  }
}

template <class Tile, int ODT>
static int launch_t(const A2aGemmArgs& a, bool fused, hipStream_t s) {
  if (a.C > 0) {
    hipLaunchKernelGGL(a2g_count_kernel, dim3((unsigned)a.C), dim3(kA2gChunk), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(a2g_scan_kernel, dim3(1), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nscatter = (int64_t)a.E * kA2gPadPieces + a.C;
  auto run = [&](auto kern, int64_t work) -> hipError_t {
    int grid = 0;
    hipError_t r = persistent_grid(reinterpret_cast<const void*>(kern), Tile::NT, work, &grid);
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(Tile::NT), 0, s, a);
    return hipGetLastError();
  };
  if (fused) return run(&a2a_gemm_kernel<Tile, ODT, true, true>, nscatter + a.max_tiles);
  if ((e = run(&a2a_gemm_kernel<Tile, ODT, true, false>, nscatter)) != hipSuccess) return e;
  return run(&a2a_gemm_kernel<Tile, ODT, false, true>, a.max_tiles);
}

int launch_a2a_gemm(const A2aGemmArgs& a, bool fused, hipStream_t s) {
  if (a.tile_m == 256)
    return a.out_dt == kBF16 ? launch_t<TileBf16Direct<256, 256, 2, 2>, kBF16>(a, fused, s)
                             : launch_t<TileBf16Direct<256, 256, 2, 2>, kF32>(a, fused, s);
  if (a.tile_m == 128 && a.out_dt == kBF16) return launch_t<TileBf16Direct<128, 256, 2, 2>, kBF16>(a, fused, s);
  return kNoKernel;
}

}  // namespace hocf
