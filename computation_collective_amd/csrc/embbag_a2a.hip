// Embedding bag + All-to-All, fused in one persistent kernel.
//
// SC24 ("Optimizing Distributed ML Communication with Fused
// Computation-Collective Operations", abstract) names embedding + All-to-All
// (the model-parallel embedding tables of DLRM) as one of its three fused
// prototypes.
//
// Work item = (table t, destination d, block j of tile_bags bags of d's
// slice).  Each half-wavefront pools one bag at a time: its 32 lanes cover
// a 512-byte row (one float4 per lane per 128 columns), the bag's indices
// are loaded once by the lanes and passed round with lane shuffles, and
// up to 24 rows (12 KB) are kept in flight before they are added -- in
// index order, from +0.0, so the result is bit-identical to a sequential
// fp32 sum.  The
// pooled row is stored straight into destination d's window at
// [slot][t][:] (512 contiguous bytes) with device-coherent stores; when the
// item's bags are stored (every thread has waited for its own) the
// workgroup stores the (t, j) flag of window d -- no L2 write-back.
//
// Items are dealt from the eight per-XCD ticket queues in table-major order,
// so each XCD works through its own eighth of the tables and keeps the
// current table's hot (Zipf-head) rows in its L2.  The kernel is a pure
// gather/stream: no matrix-core work; its roofline is HBM bandwidth.
//
// An index outside [0, R) is skipped and HOCF_ERR_BAD_INDEX recorded.
#include "internal.hpp"
#include "publish.hpp"
#include "sync.hpp"

namespace hocf {

constexpr int kEmbThreads = 256;

template <int CPL>  // float4 column slots per lane: D <= 128 * CPL
__global__ __launch_bounds__(kEmbThreads) void embbag_kernel(EmbbagArgs a) {
  // rows in flight per half-wave: 24 for rows of up to 512 bytes (a bag of
  // up to 24 lookups in one batch), fewer for wider rows (the same 12 KB in
  // flight).  Their registers set the occupancy: 24 rows keep the kernel at
  // four waves per SIMD where 32 allowed three (about 1 % faster at 20
  // lookups per bag).
  constexpr int kEmbInflight = 24 / CPL;
  __shared__ int s_qcur;
  __shared__ int64_t s_item;
  const int tid = threadIdx.x;
  const int hw = tid >> 5, hl = tid & 31;  // half-wave id, lane within it
  const int D = a.D, T = a.T, B = a.B, P = a.P;
  const int64_t R = a.R;
  const int per_t = P * a.nj;
  if (tid == 0) s_qcur = 0;
  __syncthreads();

  for (;;) {
    const int64_t item = claim_item(a.ws, a.total, &s_qcur, &s_item);
    if (item < 0) break;
    const int t = (int)(item / per_t);
    const int rem = (int)(item % per_t);
    const int d = rem / a.nj, j = rem % a.nj;
    const int s_end = min(a.Bd, (j + 1) * a.tile_bags);
    const float* tab = a.tables + (int64_t)t * R * D;
    // the item's rows of window d: slots [j * tile_bags, s_end), table t
    const __amdgpu_buffer_rsrc_t rw =
        raw_rsrc(a.win_data[d] + ((int64_t)j * a.tile_bags * T + t) * D);

    for (int s = j * a.tile_bags + hw; s < s_end; s += kEmbThreads / 32) {
      const int b = d * a.Bd + s;
      const int64_t bag = (int64_t)t * B + b;
      const int64_t lo = a.offsets ? a.offsets[bag] : bag * a.L;
      const int64_t hi = a.offsets ? a.offsets[bag + 1] : lo + a.L;
      floatx4 acc[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};

      for (int64_t base = lo; base < hi; base += 32) {
        const int n = (int)min((int64_t)32, hi - base);
        int row = -1;
        if (hl < n) {
          const int32_t ix = a.indices[base + hl];
          if (ix >= 0 && (int64_t)ix < R) row = ix;
          else report_status(a.sync, kErrBadIndex);
        }
        for (int l0 = 0; l0 < n; l0 += kEmbInflight) {
          floatx4 v[kEmbInflight][CPL];
#pragma unroll
          for (int u = 0; u < kEmbInflight; ++u) {
            const int r = __shfl(row, l0 + u, 32);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const int col = (c * 32 + hl) * 4;
              if (l0 + u < n && r >= 0 && col < D)
                v[u][c] = *reinterpret_cast<const floatx4*>(tab + (int64_t)r * D + col);
              else
                v[u][c] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
          }
          // adding +0.0 is exact here: the running sum starts at +0.0 and
          // therefore never becomes -0.0
#pragma unroll
          for (int u = 0; u < kEmbInflight; ++u)
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] = acc[c] + v[u][c];
        }
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int col = (c * 32 + hl) * 4;
        if (col < D)
          st_dev16(rw, (uint32_t)((((int64_t)(s - j * a.tile_bags) * T) * D + col) * 4), 0,
                   __builtin_bit_cast(u32x4, acc[c]));
      }
    }
    wait_memory();  // this thread's rows have completed
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(&a.win_flags[d][(int64_t)t * a.nj + j], a.sync.epoch, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  finish_workgroup(a.ws);
}

template <int CPL>
static int launch_cpl(const EmbbagArgs& a, hipStream_t s) {
  const void* k = reinterpret_cast<const void*>(&embbag_kernel<CPL>);
  int grid = 0;
  hipError_t e = persistent_grid(k, kEmbThreads, a.total, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((embbag_kernel<CPL>), dim3(grid), dim3(kEmbThreads), 0, s, a);
  return hipGetLastError();
}

int launch_embbag_a2a(const EmbbagArgs& a, hipStream_t s) {
  if (a.D <= 128) return launch_cpl<1>(a, s);
  if (a.D <= 256) return launch_cpl<2>(a, s);
  if (a.D <= 512) return launch_cpl<4>(a, s);
  return kNoKernel;
}

}  // namespace hocf
