// Flag protocol and persistent-workgroup scheduling.
//
// Producer side: a workgroup stores a tile with device-coherent stores,
// every thread waits for its own (publish.hpp), the workgroup meets at a
// barrier, and one thread stores the epoch into the tile's flag word -- no
// fence, so no L2 write-back.  Consumer side: one thread reads the flag (or
// an arrival count that is only advanced after the flags it covers) until
// it equals the epoch, the workgroup meets at a barrier, and the tile is
// read with device-coherent loads.  Flags written from outside the kernel
// (by the host or a stream write) are read at system scope and followed by
// a system-scope acquire before the data they announce is read.
//
// The pages (SC24 abstract; mKernel, section on persistent kernels and
// tile/chunk overlap) prescribe GPU-initiated, tile-granular publication but
// no memory-ordering scheme; this epoch/flag protocol is this library's.
#pragma once

#include "common.hpp"

namespace hocf {

// Values broadcast through LDS are the same in every lane, but the compiler
// cannot know it; loops and branches that depend on them must be marked
// wave-uniform, or the control-flow structurizer may split a persistent
// loop per lane (e.g. peel thread 0's flag release out of the loop), which
// breaks the barriers inside it.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void report_status(const SyncArgs& s, uint32_t code) {
  if (s.status) atomicCAS(s.status, 0u, code);
}

__device__ __forceinline__ uint32_t load_flag_agent(const uint32_t* flag) {
  return __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_flag_system(const uint32_t* flag) {
  return __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ void acquire_system() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, ""); }

// Ticket counters live in the caller's workspace:
//   ws[0 .. kNumQueues-1]  one claim counter per queue
//   ws[kNumQueues]         count of workgroups that have finished
//   ws[kNumQueues+1 ..]    operator-specific counters (reset by their users)
constexpr int kWsDone = kNumQueues;
constexpr int kWsExtra = kNumQueues + 1;

// Queue q holds the contiguous work range [qbeg(q), qbeg(q+1)) of `total`
// items.  A workgroup drains its home queue (blockIdx mod 8: workgroups are
// dispatched to the XCDs round-robin, so a queue's items share one XCD's L2)
// and then steals from the others in order.
__device__ __forceinline__ int64_t queue_begin(int q, int64_t total) {
  return (total * q) / kNumQueues;
}

// Claims the next item for this workgroup, or returns -1 when every queue is
// empty.  Must be called by all threads of the workgroup (thread 0 claims,
// the result is broadcast through LDS).  `qcur` is per-workgroup state
// (shared memory) that starts at 0.
//
// The leading barrier keeps thread 0's claim from sitting next to any
// thread-0-only code at the end of the previous item (a flag release):
// two such regions back to back get merged across the loop edge, and the
// structurizer then runs the rest of the loop without lane 0.
__device__ __forceinline__ int64_t claim_item(uint32_t* ws, int64_t total, int* s_qcur,
                                              int64_t* s_item) {
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t got = -1;
    const int home = (int)(blockIdx.x % kNumQueues);
    while (*s_qcur < kNumQueues) {
      const int q = (home + *s_qcur) % kNumQueues;
      const int64_t b = queue_begin(q, total), e = queue_begin(q + 1, total);
      const uint32_t t = __hip_atomic_fetch_add(&ws[q], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      if ((int64_t)t < e - b) { got = b + t; break; }
      ++*s_qcur;
    }
    *s_item = got;
  }
  __syncthreads();
  const int64_t it = uniform64(*s_item);
  __syncthreads();
  return it;
}

// Thread-0 state of a workgroup that claims its items one ticket ahead:
// when an item is handed out, the ticket for the next one is requested at
// once, so that request's round trip overlaps the current item's work
// instead of opening the next iteration.  Same queues and the same order of
// queues as claim_item; a ticket requested ahead is always resolved by the
// next call (a workgroup calls next() until it returns -1).
struct ClaimAhead {
  int qoff = 0;          // queues exhausted so far (home queue first)
  bool ahead = false;    // a ticket request on queue (home + qoff) is in flight
  uint32_t ticket = 0;

  __device__ __forceinline__ int64_t next(uint32_t* ws, int64_t total) {
    const int home = (int)(blockIdx.x % kNumQueues);
    int64_t got = -1;
    while (qoff < kNumQueues) {
      const int q = (home + qoff) % kNumQueues;
      const int64_t b = queue_begin(q, total), e = queue_begin(q + 1, total);
      const uint32_t t = ahead ? ticket
                               : __hip_atomic_fetch_add(&ws[q], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ahead = false;
      if ((int64_t)t < e - b) { got = b + t; break; }
      ++qoff;
    }
    if (got >= 0) {
      ticket = __hip_atomic_fetch_add(&ws[(home + qoff) % kNumQueues], 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      ahead = true;
    }
    return got;
  }
};

// Every workgroup calls this once when it has stopped claiming.  The last
// one resets the queue counters and the done counter, leaving the workspace
// zeroed for the next call (stream order makes the reset visible to it).
__device__ __forceinline__ void finish_workgroup(uint32_t* ws) {
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&ws[kWsDone], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      for (int q = 0; q < kNumQueues; ++q)
        __hip_atomic_store(&ws[q], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ws[kWsDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// As finish_workgroup, called by every thread; returns (wave-uniform, in
// every thread) whether this is the last workgroup to finish, which may then
// reset operator-specific workspace words (every other workgroup is done).
__device__ __forceinline__ bool finish_workgroup_last(uint32_t* ws, int* s_flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&ws[kWsDone], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == gridDim.x - 1;
    if (last) {
      for (int q = 0; q < kNumQueues; ++q)
        __hip_atomic_store(&ws[q], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ws[kWsDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *s_flag = last;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_flag) != 0;
}

__device__ __forceinline__ uint64_t now_ticks() { return (uint64_t)wall_clock64(); }

// Bounded wait state: deadline in wall_clock64() ticks.
struct Deadline {
  uint64_t start, ticks;
  __device__ __forceinline__ bool expired() const { return now_ticks() - start > ticks; }
};

// Whether the caller has asked every wait to stop (the abort word, read at
// system scope: the host may write it while the kernel runs).
__device__ __forceinline__ bool abort_requested(const SyncArgs& s) {
  return s.abort_flag && load_flag_system(s.abort_flag) != 0u;
}

// Outcome of a bounded wait.
enum WaitResult : int { kWaitOk = 0, kWaitTimeout = 1, kWaitAborted = 2 };

// Records the error a failed wait stands for (first writer wins).
__device__ __forceinline__ void report_wait(const SyncArgs& s, int w) {
  if (w == kWaitTimeout) report_status(s, kErrTimeout);
  else if (w == kWaitAborted) report_status(s, kErrAborted);
}

// A flag that must already hold `epoch` (its producer stored it before the
// arrival count that led here, but without waiting for that store): read
// again, with a bounded wait that also stops on an abort request, until it
// does.  kWaitOk once it does; otherwise why the wait ended.
__device__ __forceinline__ int flag_reaches(const uint32_t* flag, uint32_t seen, const SyncArgs& s) {
  if (seen == s.epoch) return kWaitOk;
  const Deadline dl{now_ticks(), s.timeout_ticks};
  for (;;) {
    __builtin_amdgcn_s_sleep(2);
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == s.epoch) return kWaitOk;
    if (abort_requested(s)) return kWaitAborted;
    if (dl.expired()) return kWaitTimeout;
  }
}

// As flag_reaches, reporting a flag that never arrives: a producer counted
// itself without storing its flag is a protocol error (on a timeout), an
// abort request is reported as such.
__device__ __forceinline__ void expect_flag(const uint32_t* flag, uint32_t seen, const SyncArgs& s) {
  const int w = flag_reaches(flag, seen, s);
  if (w == kWaitTimeout) report_status(s, kErrProtocol);
  else if (w == kWaitAborted) report_status(s, kErrAborted);
}

}  // namespace hocf
