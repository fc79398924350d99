// Device-side basics shared by the hocf kernels: vector types, bfloat16
// encoding, and the launch-argument structs the host fills in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hocf {

constexpr int kMaxP = 16;      // largest shard count (matches HOCF_MAX_P)
constexpr int kNumQueues = 8;  // one ticket queue per XCD (MI355X has 8)

// A permutation of the workgroup indices [0, grid) that gives the
// workgroups of one XCD (dispatched round-robin: XCD = index mod 8) one
// contiguous run of positions, so the work they take first is adjacent and
// shares operands in that XCD's L2.  Identity when grid is not a multiple
// of 8 (still a permutation: correctness never depends on the placement).
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t b, uint32_t grid) {
  if (grid % kNumQueues) return b;
  return (b % kNumQueues) * (grid / kNumQueues) + b / kNumQueues;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

enum Dt : int { kF32 = 0, kBF16 = 1 };

// Buffer resource word 3 for raw (untyped, 32-bit format) buffer accesses.
constexpr int kRawBufferWord3 = 0x00020000;

// A raw buffer resource over [base, base + 2 GiB).  `base` must be
// wave-uniform (it lands in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, kRawBufferWord3);
}

// bfloat16 is the top half of a binary32 pattern.
__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// binary32 -> bfloat16 with the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t r = __builtin_convertvector(floatx2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// Compile-time-typed vector access: 4 consecutive elements as fp32.
template <int DT>
__device__ __forceinline__ floatx4 ld4(const void* base, int64_t i) {
  floatx4 r;
  if constexpr (DT == kBF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + i);
    r[0] = bf16_to_f32(u.x & 0xffffu);
    r[1] = bf16_to_f32(u.x >> 16);
    r[2] = bf16_to_f32(u.y & 0xffffu);
    r[3] = bf16_to_f32(u.y >> 16);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + i);
    r[0] = f.x; r[1] = f.y; r[2] = f.z; r[3] = f.w;
  }
  return r;
}

template <int DT>
__device__ __forceinline__ void st4(void* base, int64_t i, floatx4 v) {
  if constexpr (DT == kBF16) {
    uint2 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + i) = u;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <int DT>
__device__ __forceinline__ float ld1(const void* base, int64_t i) {
  if constexpr (DT == kBF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  else return reinterpret_cast<const float*>(base)[i];
}

template <int DT>
__device__ __forceinline__ void st1(void* base, int64_t i, float v) {
  if constexpr (DT == kBF16) reinterpret_cast<uint16_t*>(base)[i] = (uint16_t)f32_to_bf16(v);
  else reinterpret_cast<float*>(base)[i] = v;
}

// The lane index, opaque to the optimiser: addresses derived from it are
// recomputed where they are used instead of being hoisted out of a
// persistent loop and held in (or spilled from) registers across it.
__device__ __forceinline__ int opaque_lane() {
  int l = (int)(threadIdx.x & 63);
  __asm__ volatile("" : "+v"(l));
  return l;
}

// Status codes the kernels record (values of hocf_status).
constexpr uint32_t kErrTimeout = 4, kErrAborted = 5, kErrBadIndex = 6, kErrProtocol = 7, kErrCapacity = 8;

// Synchronisation arguments common to every kernel.
struct SyncArgs {
  uint32_t epoch;
  uint32_t* status;            // nullable device word
  const uint32_t* abort_flag;  // nullable
  uint64_t timeout_ticks;      // in wall_clock64() ticks
};

}  // namespace hocf
