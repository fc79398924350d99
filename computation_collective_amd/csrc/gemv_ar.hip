// GEMV + AllReduce, fused in one kernel.
//
// SC24 ("Optimizing Distributed ML Communication with Fused
// Computation-Collective Operations", abstract) names GEMV + AllReduce as
// one of its three fused prototypes (the decode-time projection of a
// tensor-parallel Transformer).
//
// Work item = (shard p, column tile j): the partial y_p[:, tile] = x_p .
// W_p[:, tile] over all K, streamed from HBM once with 16-byte loads and
// fp32 FMAs on the vector ALUs (a GEMV has 4 flops per weight byte pair --
// no matrix-core work to win, the roofline is HBM).  Thread layout: TN/8
// column groups of 8 columns x (256 / (TN/8)) k-lanes; each thread keeps
// Mb x 8 accumulators; the k-lanes are folded through LDS in a fixed order.
//
// The partial is published to part[p] with a ready flag; the last of the P
// producers of column tile j (an arrival counter) folds the P partials in
// rank order in fp32, rounds once, and writes the same bits into all P
// receive windows, releasing each window's flag.  Partials and window data
// move with device-coherent 16- or 8-byte stores and loads, each writer
// waiting for its stores before the flag or count that announces them
// (publish.hpp), so no L2-wide write-back or invalidate is needed.
#include "internal.hpp"
#include "publish.hpp"
#include "sync.hpp"

namespace hocf {

constexpr int kGemvThreads = 256;
constexpr int kGemvKC = 1024;  // rows of x staged in LDS per pass
constexpr int kGemvU = 16;     // weight rows per load batch (two batches in flight)

// 4 consecutive fp32 values as SDT at byte offset off of a device-coherent resource
template <int DT>
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx4 v) {
  if constexpr (DT == kBF16) {
    const u32x2 u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(u, r, (int)off, 0, kPolicyDevice);
  } else {
    st_dev16(r, off, 0, __builtin_bit_cast(u32x4, v));
  }
}
template <int DT>
__device__ __forceinline__ floatx4 ld_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (DT == kBF16) {
    const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicyDevice);
    return floatx4{bf16_to_f32(u[0] & 0xffffu), bf16_to_f32(u[0] >> 16), bf16_to_f32(u[1] & 0xffffu),
                   bf16_to_f32(u[1] >> 16)};
  } else {
    return __builtin_bit_cast(floatx4, ld_dev16(r, off, 0));
  }
}

// Folds the P partials of column tile j in rank order in fp32, rounds once
// and stores the same bits into all P windows (device-coherent stores; the
// caller waits for them before announcing the tile).
template <int MB, int TN, int SDT, int ODT>
__device__ __forceinline__ void fold_column_tile(const GemvArArgs& a, int j) {
  constexpr int NQ = MB * TN / 4;
  constexpr int SES = SDT == kBF16 ? 2 : 4, OES = ODT == kBF16 ? 2 : 4;
  const int tid = threadIdx.x, N = a.N, P = a.P, Mb = a.Mb;
  const int n0 = j * TN, cols_valid = min(TN, N - n0);
  for (int e = tid; e < NQ; e += kGemvThreads) {
    const int qb = e / (TN / 4), qc = (e % (TN / 4)) * 4;
    if (qb >= Mb || qc >= cols_valid) continue;
    const uint32_t qoff = (uint32_t)(qb * N + n0 + qc);  // element offset in a [Mb][N] array
    floatx4 v[kMaxP];
#pragma unroll
    for (int q = 0; q < kMaxP; ++q) {
      const int qq = q < P ? q : P - 1;  // loads stay unconditional; slots past P are not added
      v[q] = ld_dev4<SDT>(raw_rsrc(reinterpret_cast<char*>(a.part) + (int64_t)qq * Mb * N * SES), qoff * SES);
    }
    floatx4 s = v[0];
#pragma unroll
    for (int q = 1; q < kMaxP; ++q)
      if (q < P) s = s + v[q];
    for (int q = 0; q < P; ++q) st_dev4<ODT>(raw_rsrc(a.win_data[q]), qoff * OES, s);
  }
}

// FUSED: the operator (publish the partial with its flag; the last producer
// of a column tile folds it).  Not FUSED: the unfused baseline's first
// kernel, which only publishes the partials.
template <int MB, int TN, int SDT, int ODT, bool FUSED>
__device__ __forceinline__ void gemv_body(const GemvArArgs& a) {
  constexpr int NCG = TN / 8;               // 16-byte column groups
  constexpr int KL = kGemvThreads / NCG;    // k-lanes
  constexpr int U = kGemvU;
  constexpr int XS_BYTES = kGemvKC * MB * 4;
  constexpr int RED_BYTES = KL * MB * TN * 4;
  static_assert(NCG * KL == kGemvThreads, "thread layout");
  constexpr int NQ = MB * TN / 4;            // output quads (4 columns of one row) per tile
  // x staging [k][MB] during the row loop, k-lane fold [KL][MB][TN] after it
  __shared__ __attribute__((aligned(16))) float lds[(XS_BYTES > RED_BYTES ? XS_BYTES : RED_BYTES) / 4];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int cg = tid % NCG, kl = tid / NCG;
  const int N = a.N, K = a.K, P = a.P, Mb = a.Mb;
  constexpr int SES = SDT == kBF16 ? 2 : 4;
  uint32_t* grp = a.ws + kWsExtra;

  for (int64_t item = blockIdx.x; item < a.total; item += gridDim.x) {
    // shard-minor numbering: with P = 8 the workgroups of one XCD (dispatched
    // round-robin, XCD = index mod 8) all stream the same shard's weights,
    // which measures about 3 % faster than spreading every shard over all XCDs
    const int p = (int)(item % P), j = (int)(item / P);
    const int n0 = j * TN;
    const int cols_valid = min(TN, N - n0);
    const bool col_ok = cg * 8 < cols_valid;
    // columns of a ragged tile's idle groups are clamped to a valid one (loaded, never used)
    const uint16_t* Wp = a.W + (int64_t)p * K * N + n0 + min(cg * 8, cols_valid - 8);
    const uint16_t* xp = a.x + (int64_t)p * Mb * K;

    float acc[MB][8];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[b][c] = 0.0f;

    for (int kc = 0; kc < K; kc += kGemvKC) {
      const int kn = min(kGemvKC, K - kc);
      // this thread's rows: kl, kl + KL, ..., two batches of U loads in flight
      const int nr = (col_ok && kl < kn) ? (kn - kl + KL - 1) / KL : 0;
      const uint16_t* w0 = Wp + (int64_t)kc * N;
      uint4 wa[U], wb[U];
      // unconditional loads (a guarded load becomes a branch and a full wait):
      // rows past this thread's last are clamped to row kn-1, loaded and not used
      auto load = [&](uint4 (&w)[U], int i0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k = min(kl + (i0 + u) * KL, kn - 1);
          w[u] = *reinterpret_cast<const uint4*>(w0 + (int64_t)k * N);
        }
      };
      auto consume = [&](const uint4 (&w)[U], int i0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (i0 + u >= nr) break;
          const int k = kl + (i0 + u) * KL;
          float xv[MB];
          if constexpr (MB % 4 == 0) {
#pragma unroll
            for (int b = 0; b < MB; b += 4) {
              const floatx4 t = *reinterpret_cast<const floatx4*>(&lds[k * MB + b]);
              xv[b] = t[0]; xv[b + 1] = t[1]; xv[b + 2] = t[2]; xv[b + 3] = t[3];
            }
          } else {
#pragma unroll
            for (int b = 0; b < MB; ++b) xv[b] = lds[k * MB + b];
          }
          const uint32_t wd[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float lo = bf16_to_f32(wd[c] & 0xffffu), hi = bf16_to_f32(wd[c] >> 16);
#pragma unroll
            for (int b = 0; b < MB; ++b) {
              acc[b][2 * c] = fmaf(xv[b], lo, acc[b][2 * c]);
              acc[b][2 * c + 1] = fmaf(xv[b], hi, acc[b][2 * c + 1]);
            }
          }
        }
      };
      // x first (16-byte pieces x[b][k .. k+7]), then the first batch of
      // weight rows, the second once x is in LDS: the vector-memory counter
      // completes in issue order, so the wait for x includes no weight load,
      // and x does not queue behind a full double batch of them
      constexpr int XL = (MB * kGemvKC / 8 + kGemvThreads - 1) / kGemvThreads;
      const int npc = kn / 8;  // 16-byte pieces per row of x in this pass
      uint4 xr[XL];
#pragma unroll
      for (int t = 0; t < XL; ++t) {  // pieces past x's end are clamped to its last piece (not used)
        const int e = min(tid + t * kGemvThreads, Mb * npc - 1);
        xr[t] = *reinterpret_cast<const uint4*>(xp + (int64_t)(e / npc) * K + kc + (e % npc) * 8);
      }
      load(wa, 0);
      lds_barrier();  // the previous pass (or item) is done with lds
#pragma unroll
      for (int t = 0; t < XL; ++t) {
        const int e = tid + t * kGemvThreads, b = e / npc, k0 = (e % npc) * 8;
        if (e < MB * npc) {
          const uint32_t wd[4] = {xr[t].x, xr[t].y, xr[t].z, xr[t].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            lds[(k0 + 2 * c) * MB + b] = b < Mb ? bf16_to_f32(wd[c] & 0xffffu) : 0.0f;
            lds[(k0 + 2 * c + 1) * MB + b] = b < Mb ? bf16_to_f32(wd[c] >> 16) : 0.0f;
          }
        }
      }
      lds_barrier();
      load(wb, U);
      for (int i0 = 0; i0 < nr; i0 += 2 * U) {
        consume(wa, i0);
        load(wa, i0 + 2 * U);
        consume(wb, i0 + U);
        load(wb, i0 + 3 * U);
      }
    }

    // fold the k-lanes in order kl = 0..KL-1, one output quad per thread
    lds_barrier();  // every thread is done reading x from lds
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int c = 0; c < 8; c += 4)
        *reinterpret_cast<floatx4*>(&lds[(kl * MB + b) * TN + cg * 8 + c]) =
            floatx4{acc[b][c], acc[b][c + 1], acc[b][c + 2], acc[b][c + 3]};
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rpart = raw_rsrc(reinterpret_cast<char*>(a.part) + (int64_t)p * Mb * N * SES);
    for (int e = tid; e < NQ; e += kGemvThreads) {
      const int qb = e / (TN / 4), qc = (e % (TN / 4)) * 4;  // row, first column of the quad
      if (qb >= Mb || qc >= cols_valid) continue;
      floatx4 s = *reinterpret_cast<const floatx4*>(&lds[qb * TN + qc]);
      for (int q = 1; q < KL; ++q) s = s + *reinterpret_cast<const floatx4*>(&lds[(q * MB + qb) * TN + qc]);
      st_dev4<SDT>(rpart, (uint32_t)(qb * N + n0 + qc) * SES, s);
    }
    if constexpr (!FUSED) {
      __syncthreads();  // the fold's lds reads are done before the next item stages x
      continue;
    }
    wait_memory();
    __syncthreads();

    // ready flag; arrival count -> the last producer of tile j reduces
    if (tid == 0) {
      // (the partial is complete; the reducer re-reads the flag, bounded, if
      // it gets there before the flag store has)
      __hip_atomic_store(&a.part_flags[(int64_t)p * a.ntiles + j], a.sync.epoch, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      uint32_t* cnt = &grp[j];
      const uint32_t prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = (prev == (uint32_t)(P - 1));
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (uniform(s_last)) {
      // the count says every partial of tile j has landed (each producer
      // waited for its stores before counting), so the fold's loads need not
      // wait for the flags: they are read first and checked after the fold
      const uint32_t* f = &a.part_flags[(int64_t)min(tid, P - 1) * a.ntiles + j];
      const uint32_t seen = tid < P ? load_flag_agent(f) : a.sync.epoch;
      fold_column_tile<MB, TN, SDT, ODT>(a, j);
      if (tid < P) expect_flag(f, seen, a.sync);
      wait_memory();
      __syncthreads();
      if (tid < P)
        __hip_atomic_store(&a.win_flags[tid][j], a.sync.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Two workgroups per CU where the registers allow (up to 4 batch rows); with
// 5 to 8 rows the accumulators and the two load batches need more than the
// 128 registers two workgroups per CU leave, so those run one per CU rather
// than spill to scratch.
constexpr int gemv_wgs_per_cu(int mb) { return mb <= 4 ? 2 : 1; }

template <int MB, int TN, int SDT, int ODT>
__global__ __launch_bounds__(kGemvThreads, gemv_wgs_per_cu(MB)) void gemv_ar_kernel(GemvArArgs a) {
  gemv_body<MB, TN, SDT, ODT, true>(a);
}

// The unfused baseline: the GEMV publishing its partials and nothing else ...
template <int MB, int TN, int SDT, int ODT>
__global__ __launch_bounds__(kGemvThreads, gemv_wgs_per_cu(MB)) void unfused_gemv_kernel(GemvArArgs a) {
  gemv_body<MB, TN, SDT, ODT, false>(a);
}

// ... then, after it (stream order), one workgroup per column tile folds the
// P partials and writes the result into all P windows.
template <int MB, int TN, int SDT, int ODT>
__global__ __launch_bounds__(kGemvThreads) void unfused_gemv_fold_kernel(GemvArArgs a) {
  fold_column_tile<MB, TN, SDT, ODT>(a, (int)blockIdx.x);
}

template <int MB, int TN, int SDT, int ODT>
static int launch_k(const GemvArArgs& a, hipStream_t s) {
  auto kern = a.fused ? &gemv_ar_kernel<MB, TN, SDT, ODT> : &unfused_gemv_kernel<MB, TN, SDT, ODT>;
  int grid = 0;
  hipError_t e = persistent_grid(reinterpret_cast<const void*>(kern), kGemvThreads, a.total, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemvThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.fused) return e;
  hipLaunchKernelGGL((unfused_gemv_fold_kernel<MB, TN, SDT, ODT>), dim3(a.ntiles), dim3(kGemvThreads), 0, s, a);
  return hipGetLastError();
}

template <int MB, int TN>
static int launch_dt(const GemvArArgs& a, hipStream_t s) {
  if (a.slot_dt == kF32 && a.out_dt == kBF16) return launch_k<MB, TN, kF32, kBF16>(a, s);
  if (a.slot_dt == kBF16 && a.out_dt == kBF16) return launch_k<MB, TN, kBF16, kBF16>(a, s);
  if (a.slot_dt == kF32 && a.out_dt == kF32) return launch_k<MB, TN, kF32, kF32>(a, s);
  return launch_k<MB, TN, kBF16, kF32>(a, s);
}

template <int TN>
static int launch_tn(const GemvArArgs& a, hipStream_t s) {
  if (a.Mb <= 1) return launch_dt<1, TN>(a, s);
  if (a.Mb <= 2) return launch_dt<2, TN>(a, s);
  if (a.Mb <= 4) return launch_dt<4, TN>(a, s);
  return launch_dt<8, TN>(a, s);
}

int launch_gemv_ar(const GemvArArgs& a, hipStream_t s) {
  switch (a.tile_n) {
    case 128: return launch_tn<128>(a, s);
    case 256: return launch_tn<256>(a, s);
    case 512: return launch_tn<512>(a, s);
  }
  return kNoKernel;
}

}  // namespace hocf
