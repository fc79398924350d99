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
// receive windows, releasing each window's flag.
#include "internal.hpp"
#include "sync.hpp"

namespace hocf {

constexpr int kGemvThreads = 256;
constexpr int kGemvKC = 512;  // rows of x staged in LDS per pass
constexpr int kGemvUnroll = 16;

template <int MB, int TN, int SDT, int ODT>
__global__ __launch_bounds__(kGemvThreads) void gemv_ar_kernel(GemvArArgs a) {
  constexpr int NCG = TN / 8;               // column groups
  constexpr int KL = kGemvThreads / NCG;    // k-lanes
  static_assert(NCG * KL == kGemvThreads, "thread layout");
  __shared__ float xs[MB][kGemvKC];
  __shared__ float red[KL][MB][TN];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int cg = tid % NCG, kl = tid / NCG;
  const int N = a.N, K = a.K, P = a.P, Mb = a.Mb;
  uint32_t* grp = a.ws + kWsExtra;

  for (int64_t item = blockIdx.x; item < a.total; item += gridDim.x) {
    const int p = (int)(item / a.ntiles), j = (int)(item % a.ntiles);
    const int n0 = j * TN;
    const int cols_valid = min(TN, N - n0);
    const int ncol = n0 + cg * 8;
    const bool col_ok = cg * 8 < cols_valid;
    const uint16_t* Wp = a.W + (int64_t)p * K * N + ncol;
    const uint16_t* xp = a.x + (int64_t)p * Mb * K;

    float acc[MB][8];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[b][c] = 0.0f;

    for (int kc = 0; kc < K; kc += kGemvKC) {
      const int kn = min(kGemvKC, K - kc);
      __syncthreads();
      for (int e = tid; e < MB * kGemvKC; e += kGemvThreads) {
        const int b = e / kGemvKC, k = e % kGemvKC;
        xs[b][k] = (b < Mb && k < kn) ? bf16_to_f32(xp[(int64_t)b * K + kc + k]) : 0.0f;
      }
      __syncthreads();
      if (col_ok) {
        // rows kl, kl + KL, ... of this pass, kGemvUnroll loads in flight
        for (int k0 = kl; k0 < kn; k0 += KL * kGemvUnroll) {
          uint4 w[kGemvUnroll];
#pragma unroll
          for (int u = 0; u < kGemvUnroll; ++u) {
            const int k = k0 + u * KL;
            w[u] = k < kn ? *reinterpret_cast<const uint4*>(Wp + (int64_t)(kc + k) * N)
                          : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < kGemvUnroll; ++u) {
            const int k = k0 + u * KL;
            if (k < kn) {
              const uint32_t wd[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
              for (int b = 0; b < MB; ++b) {
                const float xv = xs[b][k];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                  acc[b][2 * c] = fmaf(xv, bf16_to_f32(wd[c] & 0xffffu), acc[b][2 * c]);
                  acc[b][2 * c + 1] = fmaf(xv, bf16_to_f32(wd[c] >> 16), acc[b][2 * c + 1]);
                }
              }
            }
          }
        }
      }
    }

    // fold the k-lanes in order kl = 0..KL-1
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c) red[kl][b][cg * 8 + c] = acc[b][c];
    __syncthreads();
    const int64_t pstride = (int64_t)Mb * N;
    for (int e = tid; e < MB * TN; e += kGemvThreads) {
      const int b = e / TN, col = e % TN;
      if (b < Mb && col < cols_valid) {
        float s = red[0][b][col];
        for (int q = 1; q < KL; ++q) s += red[q][b][col];
        st1<SDT>(a.part, p * pstride + (int64_t)b * N + n0 + col, s);
      }
    }
    __syncthreads();

    if (tid == 0) {
      release_flag(&a.part_flags[(int64_t)p * a.ntiles + j], a.sync.epoch);
      uint32_t* cnt = &grp[j];
      const uint32_t prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const int last = (prev == (uint32_t)(P - 1));
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (uniform(s_last)) {
      acquire_agent();
      if (tid < P && load_flag_agent(&a.part_flags[(int64_t)tid * a.ntiles + j]) != a.sync.epoch)
        report_status(a.sync, kErrProtocol);
      for (int e = tid; e < Mb * TN; e += kGemvThreads) {
        const int b = e / TN, col = e % TN;
        if (col >= cols_valid) continue;
        const int64_t off = (int64_t)b * N + n0 + col;
        float v[kMaxP];
#pragma unroll
        for (int q = 0; q < kMaxP; ++q)
          if (q < P) v[q] = ld1<SDT>(a.part, q * pstride + off);
        float s = v[0];
#pragma unroll
        for (int q = 1; q < kMaxP; ++q)
          if (q < P) s += v[q];
        for (int q = 0; q < P; ++q) st1<ODT>(a.win_data[q], off, s);
      }
      __syncthreads();
      if (tid < P) release_flag(&a.win_flags[tid][j], a.sync.epoch);
    }
    __syncthreads();
  }
}

template <int MB, int TN, int SDT, int ODT>
static hipError_t launch_k(const GemvArArgs& a, hipStream_t s) {
  auto kern = &gemv_ar_kernel<MB, TN, SDT, ODT>;
  int grid = 0;
  hipError_t e = persistent_grid(reinterpret_cast<const void*>(kern), kGemvThreads, a.total, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemvThreads), 0, s, a);
  return hipGetLastError();
}

template <int MB, int TN>
static hipError_t launch_dt(const GemvArArgs& a, hipStream_t s) {
  if (a.slot_dt == kF32 && a.out_dt == kBF16) return launch_k<MB, TN, kF32, kBF16>(a, s);
  if (a.slot_dt == kBF16 && a.out_dt == kBF16) return launch_k<MB, TN, kBF16, kBF16>(a, s);
  if (a.slot_dt == kF32 && a.out_dt == kF32) return launch_k<MB, TN, kF32, kF32>(a, s);
  return launch_k<MB, TN, kBF16, kF32>(a, s);
}

template <int TN>
static hipError_t launch_tn(const GemvArArgs& a, hipStream_t s) {
  if (a.Mb <= 1) return launch_dt<1, TN>(a, s);
  if (a.Mb <= 2) return launch_dt<2, TN>(a, s);
  if (a.Mb <= 4) return launch_dt<4, TN>(a, s);
  return launch_dt<8, TN>(a, s);
}

hipError_t launch_gemv_ar(const GemvArArgs& a, hipStream_t s) {
  switch (a.tile_n) {
    case 128: return launch_tn<128>(a, s);
    case 256: return launch_tn<256>(a, s);
    case 512: return launch_tn<512>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hocf
