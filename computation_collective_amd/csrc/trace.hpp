// Per-iteration timestamps of the GEMM + ReduceScatter / AllReduce
// persistent kernel, compiled in only when HOCF_TRACE is defined (the
// library's trace build, libhocf_trace.so); in the product library every
// call below is empty.
//
// The claim the fused kernel rests on (SC24 abstract; mKernel, section on
// persistent kernels and tile/chunk overlap) is that the collective's work
// -- here the rank-order folds of published tiles -- runs while other
// workgroups of the same kernel are still computing.  Each iteration of a
// workgroup records when it started, when its claim resolved, when its
// mainloop started and ended, when its tile's stores had completed and when
// its flag and count were done, together with the tile and band it took, so
// the fold intervals can be set against every other workgroup's mainloop
// intervals on one clock (the device's constant-rate wall clock, the same
// on every CU).
//
// Record layout (64 bytes, 8 uint64): [0..5] the six timestamps above,
// [6] the work item (-1: none), [7] the band (low 32 bits, -1: none) and
// TraceBits (high 32 bits).  Records of workgroup b, iteration i at
// ((b * kTraceIters) + i) * 64 bytes from the trace region, which the trace
// build's workspace query appends after the scheduler words (the caller
// zeroes it; unwritten records stay zero).
#pragma once

#include "common.hpp"

namespace hocf {

constexpr int kTraceIters = 64;   // records kept per workgroup
constexpr int kTraceWgs = 2048;   // workgroups recorded
constexpr int kTraceRecWords = 8;
constexpr int64_t kTraceBytes = (int64_t)kTraceIters * kTraceWgs * kTraceRecWords * 8;
#if defined(HOCF_TRACE)
constexpr bool kTraceBuild = true;
#else
constexpr bool kTraceBuild = false;
#endif

enum TracePoint : int { kTrStart = 0, kTrClaimed, kTrMainStart, kTrMainEnd, kTrStored, kTrDone, kTrPoints };
enum TraceBits : uint32_t {
  kTrBandInLoop = 1,  // the iteration's band rode along its mainloop
  kTrBandAlone = 2,   // the iteration folded its band on its own (before its mainloop, or with no tile)
  kTrCompleted = 4    // this workgroup was the last producer of its tile's output tile
};

struct TraceSink {
#if defined(HOCF_TRACE)
  uint64_t* base;
  uint64_t t[kTrPoints];  // wave-uniform: kept in scalar registers
  int iter;
  __device__ __forceinline__ void init(uint64_t* b) {
    base = b;
    iter = 0;
#pragma unroll
    for (int k = 0; k < kTrPoints; ++k) t[k] = 0;
  }
  // every thread calls it at the same point (the value is wave-uniform)
  __device__ __forceinline__ void mark(int k) { t[k] = (uint64_t)wall_clock64(); }
  // thread 0 stores the record (plain vector stores)
  __device__ __forceinline__ void commit(int64_t item, int band, uint32_t bits) {
    if (threadIdx.x == 0 && base && blockIdx.x < (unsigned)kTraceWgs && iter < kTraceIters) {
      uint64_t* r = base + ((int64_t)blockIdx.x * kTraceIters + iter) * kTraceRecWords;
#pragma unroll
      for (int k = 0; k < kTrPoints; ++k) r[k] = t[k];
      r[6] = (uint64_t)item;
      r[7] = ((uint64_t)bits << 32) | (uint32_t)band;
    }
    ++iter;
  }
#else
  __device__ __forceinline__ void init(uint64_t*) {}
  __device__ __forceinline__ void mark(int) {}
  __device__ __forceinline__ void commit(int64_t, int, uint32_t) {}
#endif
};

}  // namespace hocf
