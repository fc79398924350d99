// One workgroup computes one TM x TN output tile  C = A[rows, :] . W[:, cols]
// on the matrix cores (fp32 accumulation), staging A and W tiles through
// LDS with a two-stage pipeline: while the MFMAs consume stage s, the next
// K-slice is already in flight from global memory into registers, and is
// written to stage s^1 before the single barrier of the step.
//
// bf16 path (gfx950 v_mfma_f32_32x32x16_bf16): each lane feeds 8 consecutive
// k of one row of A and 8 consecutive k of one column of W.  A is row-major
// [M][K], so its rows are copied to LDS as they are.  W is row-major [K][N],
// so its K-slice is transposed on the way into LDS: each thread loads a
// 4(k) x 8(n) block (four 16-byte row pieces, 128-byte coalesced per 8
// lanes), regroups it in registers into eight 4(k) pieces and writes those
// into the transposed tile Wt[n][k].  LDS rows are padded to 144 bytes and
// Wt's 8-byte k-slots are XOR-swizzled by bit 4 of n, so both the
// transposing writes and the MFMA operand reads spread over all banks.
//
// fp32 path (v_mfma_f32_32x32x2f32, one element per lane and operand): no
// transpose is needed; W's K-slice is kept [k][n].
//
// The MFMA is fed with W as its first operand and A as its second, so each
// 32x32 accumulator block holds C^T: lane l, block (i, j), element v = 4g+e
// holds tile row  wm*WTM + 32i + l%32  and column  wn*WTN + 32j + 8g +
// 4(l/32) + e.  Each lane therefore owns runs of 4 consecutive columns of
// one row, which the epilogues store as 16-byte (fp32) or 8-byte (bf16)
// vectors.
#pragma once

#include <type_traits>
#include <utility>

#include "common.hpp"

namespace hocf {

__device__ __forceinline__ uint32_t u4_word(const uint4& v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

template <int TM_, int TN_, int WM_, int WN_>
struct TileBf16 {
  static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
  static constexpr bool kSplitMainloop = false;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int BK = 64;
  static constexpr int LDK = BK + 8;  // padded row: 72 bf16 = 144 bytes
  static constexpr int WTM = TM / WM, WTN = TN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_ELEMS = TM * LDK, B_ELEMS = TN * LDK, STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int SMEM_BYTES = LDS_BYTES;  // stage array 0 holds everything
  static constexpr int NST = 1;
  static constexpr int A_LD = (TM * BK / 8) / NT;  // 16-byte A pieces per thread per step
  static constexpr int NBH = TN / 64;              // W wave-blocks along n (8 lanes x 8 n)
  static constexpr int B_BLK = 2 * NBH / NW;       // 4(k) x 8(n) W blocks per thread per step
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert((TM * BK / 8) % NT == 0 && A_LD >= 1, "A slice must split evenly");
  static_assert(B_BLK >= 1 && B_BLK * NW == 2 * NBH, "W slice must split evenly over the waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  // Tile coordinates of accumulator elements acc[i][j][4g .. 4g+3]: one row, 4 columns.
  __device__ static __forceinline__ void quad(int i, int j, int g, int lane, int wave, int& row,
                                              int& col0) {
    const int wm = wave / WN, wn = wave % WN;
    row = wm * WTM + 32 * i + (lane & 31);
    col0 = wn * WTN + 32 * j + 8 * g + 4 * (lane >> 5);
  }

  // Stores the accumulators of this lane into a row-major tile at `base`
  // (leading dimension ld, element type DT): one base pointer per lane, the
  // block and group offsets are compile-time constants.
  template <int DT, bool RAGGED, int FM_, int FN_, int WTM_, int WTN_>
  __device__ static __forceinline__ void store_acc_impl(void* base, int64_t ld, int rows_valid,
                                                        int cols_valid,
                                                        const floatx16 (&acc)[FM_][FN_]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = (wave / WN) * WTM_ + (lane & 31);
    const int c0 = (wave % WN) * WTN_ + 4 * (lane >> 5);
    constexpr int ES = DT == kBF16 ? 2 : 4;
    char* p = reinterpret_cast<char*>(base) + ((int64_t)r0 * ld + c0) * ES;
#pragma unroll
    for (int i = 0; i < FM_; ++i) {
      char* pi = p + (int64_t)(32 * i) * ld * ES;
#pragma unroll
      for (int j = 0; j < FN_; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (RAGGED && (r0 + 32 * i >= rows_valid || c0 + 32 * j + 8 * g >= cols_valid)) continue;
          const floatx4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                             acc[i][j][4 * g + 3]};
          st4<DT>(pi + (32 * j + 8 * g) * ES, 0, v);
        }
      // keep the scheduler from hoisting every block's conversion at once
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  template <int DT, bool RAGGED>
  __device__ static __forceinline__ void store_acc(void* base, int64_t ld, int rows_valid,
                                                   int cols_valid, const floatx16 (&acc)[FM][FN]) {
    store_acc_impl<DT, RAGGED, FM, FN, WTM, WTN>(base, ld, rows_valid, cols_valid, acc);
  }

  // Physical 8-byte k-slot of logical slot s in Wt row n (bit 3 flipped by bit 4 of n).
  __device__ static __forceinline__ int wslot(int n, int s) { return s ^ (((n >> 4) & 1) << 3); }

  template <bool RAGGED>
  __device__ static __forceinline__ void run(const uint16_t* __restrict__ A, int64_t lda,
                                             const uint16_t* __restrict__ W, int64_t ldw,
                                             int rows_valid, int cols_valid, int K,
                                             char* const (&stages)[4], floatx16 (&acc)[FM][FN]) {
    uint16_t* const lds = reinterpret_cast<uint16_t*>(stages[0]);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // this thread's W blocks: 4 k-rows x 8 n-columns each; wave-block id
    // wave + NW*i covers n-block group (id mod NBH) and k-half (id / NBH)
    int nbv[B_BLK], kbv[B_BLK];
#pragma unroll
    for (int i = 0; i < B_BLK; ++i) {
      const int id = wave + NW * i;
      nbv[i] = (id % NBH) * 8 + (lane & 7);
      kbv[i] = (id / NBH) * 8 + (lane >> 3);
    }

    uint4 ra[A_LD];
    uint4 rb[B_BLK][4];
    const int nk = (K + BK - 1) / BK;

    auto load_global = [&](int ks) {
      const int k0 = ks * BK;
#pragma unroll
      for (int t = 0; t < A_LD; ++t) {
        const int c = tid + t * NT;
        const int row = c / (BK / 8), kc = c % (BK / 8);
        const int k = k0 + kc * 8;
        if (!RAGGED || (row < rows_valid && k < K))
          ra[t] = *reinterpret_cast<const uint4*>(A + (int64_t)row * lda + k);
        else
          ra[t] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < B_BLK; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = k0 + kbv[i] * 4 + j, n = nbv[i] * 8;
          if (!RAGGED || (k < K && n < cols_valid))
            rb[i][j] = *reinterpret_cast<const uint4*>(W + (int64_t)k * ldw + n);
          else
            rb[i][j] = make_uint4(0, 0, 0, 0);
        }
    };

    auto store_lds = [&](int stage) {
      uint16_t* As = lds + stage * STAGE;
      uint16_t* Bs = As + A_ELEMS;
#pragma unroll
      for (int t = 0; t < A_LD; ++t) {
        const int c = tid + t * NT;
        const int row = c / (BK / 8), kc = c % (BK / 8);
        *reinterpret_cast<uint4*>(As + row * LDK + kc * 8) = ra[t];
      }
      // transpose each 4x8 block: for column e, pack k = 0..3 into 8 bytes
#pragma unroll
      for (int i = 0; i < B_BLK; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = e >> 1;
          const uint32_t w0 = u4_word(rb[i][0], d), w1 = u4_word(rb[i][1], d);
          const uint32_t w2 = u4_word(rb[i][2], d), w3 = u4_word(rb[i][3], d);
          uint32_t lo, hi;
          if (e & 1) {
            lo = (w0 >> 16) | (w1 & 0xffff0000u);
            hi = (w2 >> 16) | (w3 & 0xffff0000u);
          } else {
            lo = (w0 & 0xffffu) | (w1 << 16);
            hi = (w2 & 0xffffu) | (w3 << 16);
          }
          const int n = nbv[i] * 8 + e;
          *reinterpret_cast<uint2*>(Bs + n * LDK + wslot(n, kbv[i]) * 4) = make_uint2(lo, hi);
        }
    };

    // MFMA operand fragments of one 16-deep k-slice
    auto read_frags = [&](const uint16_t* As, const uint16_t* Bs, int kk, bf16x8 (&a)[FM],
                          bf16x8 (&b)[FN]) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = wm * WTM + 32 * i + (lane & 31);
        a[i] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(As + m * LDK + kk * 16 + (lane >> 5) * 8));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * WTN + 32 * j + (lane & 31);
        const int sl = kk * 4 + (lane >> 5) * 2;
        b[j] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(Bs + n * LDK + wslot(n, sl) * 4));
      }
    };
    auto mfmas = [&](const bf16x8 (&a)[FM], const bf16x8 (&b)[FN]) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    };
    // the fragments of slice kk+1 are read while the MFMAs of slice kk run
    auto compute = [&](int stage) {
      const uint16_t* As = lds + stage * STAGE;
      const uint16_t* Bs = As + A_ELEMS;
      bf16x8 a0[FM], b0[FN], a1[FM], b1[FN];
      read_frags(As, Bs, 0, a0, b0);
#pragma unroll
      for (int kk = 0; kk < BK / 16; kk += 2) {
        read_frags(As, Bs, kk + 1, a1, b1);
        mfmas(a0, b0);
        if (kk + 2 < BK / 16) read_frags(As, Bs, kk + 2, a0, b0);
        mfmas(a1, b1);
      }
    };

    if (nk == 0) return;
    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      if (ks + 1 < nk) load_global(ks + 1);
      compute(ks & 1);
      if (ks + 1 < nk) store_lds((ks + 1) & 1);
      __syncthreads();
    }
  }
};

// Instruction-order hints for one k-substep: NM MFMAs, with ND LDS reads
// front-loaded (ceil(ND/NM) after each MFMA until they run out, so the last
// read still has MFMAs behind it) and NV global loads spread evenly.
template <int NM, int ND, int NV, int X>
__device__ __forceinline__ void interleave_step() {
  constexpr int dpm = (ND + NM - 1) / NM;
  constexpr int d = ND - X * dpm < dpm ? (ND - X * dpm > 0 ? ND - X * dpm : 0) : dpm;
  constexpr int v = (NV * (X + 1)) / NM - (NV * X) / NM;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
  if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);  // global load
  if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);  // LDS read
}
template <int NM, int ND, int NV, int... X>
__device__ __forceinline__ void interleave_impl(std::integer_sequence<int, X...>) {
  (interleave_step<NM, ND, NV, X>(), ...);
}
template <int NM, int ND, int NV>
__device__ __forceinline__ void interleave() {
  interleave_impl<NM, ND, NV>(std::make_integer_sequence<int, NM>{});
}

// Work a mainloop can carry at the ends of its K rounds (see
// TileBf16Direct::body): NPASS units, unit u's V vector-memory loads issued
// by issue(u) at the end of round u and consumed by fold(u) at the end of
// round u+1, where no vector-memory operation may be issued.
struct NoSide {
  static constexpr int NPASS = 0, V = 0;
  __device__ void issue(int) {}
  __device__ void fold(int) {}
};

// bf16 tile, full tiles only (no ragged rows, columns or K): both operands
// go from global memory straight into LDS (gfx950 global_load_lds, 16 bytes
// per lane, a wave writing 1 KB of LDS per instruction), so no registers hold
// staged data and nothing is transposed in registers.
//
// W: NST = 4 LDS stages of one 32-deep K slice ([BK][TN] rows, the kernel's
// four stage arrays), loads issued three slices ahead.  A: two double stages
// of two slices each ([TM][2*BK] rows of 128 bytes, direct_a_stage0/1).  An
// A row of a single 32-deep slice would be 64 bytes, half a cache line, and
// the vector L1 would then send two miss requests per line of A; the
// operand stream of a tile is bound by how many misses the L1 keeps in
// flight, and whole-line A requests (a third fewer requests in all) made
// GEMM+ReduceScatter 3.5 % faster.  The price: an A double stage holding
// slices (2d, 2d+1) is refilled, with slices 2d+4 and 2d+5, only after slice
// 2d+1's reads, so A's loads get about a slice and a half to land where W's
// get three.  Every stage is its own __shared__ array and the K loop is
// unrolled by four slices, so every LDS access names its array; the compiler
// then knows that reading one stage does not alias the loads still in flight
// into the others, and does not wait for them.
//
// Layouts, in 16-byte chunks XOR-swizzled on the global side (a lane may
// fetch any global address):
//   A row m, logical chunk c (of 8) -> physical chunk c ^ ((m / 2) mod 8)
//   W row k, logical chunk c -> physical chunk c ^ (4 * (k mod 4))
// A fragments are 16-byte ds_read_b128 (8 consecutive k of one row of A).
// W fragments use the gfx950 transposing read ds_read_b64_tr_b16: within a
// group of 16 lanes, lane s points at W[k0 + s/4][n0 + 4*(s%4) .. +3] and
// lane i receives W[k0 .. k0+3][n0 + i]; two such reads give the 8
// consecutive k of one column of W.  Both read patterns touch 16 distinct
// 16-byte bank groups per 16 lanes (conflict-free).
//
// Load order: the prologue issues A(0..1), W(0), W(1), A(2..3), W(2); the
// body W(3); slice j then issues W(j+4) and, for odd j, A(j+3 .. j+4).  The
// wait of slice j counts the operations issued after the last one slice
// j+1 needs: 2 W_LD + A_LD after an even slice, W_LD after an odd one, and
// 2 W_LD + A_LD, 0, 0 in the last round (the band loads a side pass adds
// in flight come on top).

// The direct tiles' two A double stages (up to 256 rows x 64 k of bf16
// each): one __shared__ array each, one definition per kernel, shared by
// every direct tile the kernel uses.
constexpr int kDirectAStageBytes = 256 * 64 * 2;
__device__ __forceinline__ char* direct_a_stage0() {
  __shared__ __attribute__((aligned(1024))) char a0[kDirectAStageBytes];
  return a0;
}
__device__ __forceinline__ char* direct_a_stage1() {
  __shared__ __attribute__((aligned(1024))) char a1[kDirectAStageBytes];
  return a1;
}

template <int TM_, int TN_, int WM_, int WN_, int BK_ = 32, int NST_ = 4>
struct TileBf16Direct {
  static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
  static constexpr bool kSplitMainloop = true;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static_assert(BK_ == 32 && NST_ == 4, "one 32-deep slice per W stage, four W stages, two A double stages");
  static constexpr int BK = BK_, NST = NST_;
  static constexpr int WTM = TM / WM, WTN = TN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A2_BYTES = TM * 2 * BK * 2;   // two slices of A, 128-byte rows
  static constexpr int W_BYTES = BK * TN * 2;
  static constexpr int SMEM_BYTES = W_BYTES;          // each of the kernel's 4 stage arrays holds one W slice
  static constexpr int LDS_BYTES = NST * W_BYTES + 2 * A2_BYTES;
  static constexpr int A_LD = A2_BYTES / 1024 / NW;   // loads per wave per A double stage
  static constexpr int W_LD = W_BYTES / 1024 / NW;    // loads per wave per W slice
  static constexpr int CA = 2 * BK / 8;               // 16-byte chunks per A row (8)
  static constexpr int AROWS_PER_BLOCK = 1024 / (2 * BK * 2);
  static constexpr int CW = TN / 8;
  static constexpr int WROWS_PER_BLOCK = 512 / TN;
  static constexpr int KSTEP = NST * BK;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert((A2_BYTES / 1024) % NW == 0 && (W_BYTES / 1024) % NW == 0 && TN >= 128 && TN <= 512, "layout");
  static_assert(A2_BYTES <= kDirectAStageBytes, "A double stage larger than the shared arrays");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  __device__ static __forceinline__ void quad(int i, int j, int g, int lane, int wave, int& row,
                                              int& col0) {
    const int wm = wave / WN, wn = wave % WN;
    row = wm * WTM + 32 * i + (lane & 31);
    col0 = wn * WTN + 32 * j + 8 * g + 4 * (lane >> 5);
  }

  template <int DT, bool RAGGED>
  __device__ static __forceinline__ void store_acc(void* base, int64_t ld, int rows_valid,
                                                   int cols_valid, const floatx16 (&acc)[FM][FN]) {
    TileBf16<TM, TN, WM, WN>::template store_acc_impl<DT, RAGGED, FM, FN, WTM, WTN>(
        base, ld, rows_valid, cols_valid, acc);
  }

  template <bool RAGGED>
  __device__ static __forceinline__ void run(const uint16_t* __restrict__ A, int64_t lda,
                                             const uint16_t* __restrict__ W, int64_t ldw,
                                             int rows_valid, int cols_valid, int K,
                                             char* const (&stages)[4], floatx16 (&acc)[FM][FN]) {
    NoSide none;
    parts<RAGGED, true, true>(A, lda, W, ldw, rows_valid, cols_valid, K, stages, acc, none);
  }
  // Split use: prologue() issues the loads of the first slices (A(0..3),
  // W(0..2)) and returns; body() (same arguments) then issues W(3) and runs
  // the K loop.  Between the two the workgroup may do anything that leaves
  // the stage arrays alone: vector-memory operations it issues meanwhile only
  // make body()'s first wait (counted from the end) wait longer.
  __device__ static __forceinline__ void prologue(const uint16_t* __restrict__ A, int64_t lda,
                                                  const uint16_t* __restrict__ W, int64_t ldw, int K,
                                                  char* const (&stages)[4]) {
    floatx16 unused[FM][FN];
    NoSide none;
    parts<false, true, false>(A, lda, W, ldw, TM, TN, K, stages, unused, none);
  }
  template <bool RAGGED>
  __device__ static __forceinline__ void body(const uint16_t* __restrict__ A, int64_t lda,
                                              const uint16_t* __restrict__ W, int64_t ldw,
                                              int rows_valid, int cols_valid, int K,
                                              char* const (&stages)[4], floatx16 (&acc)[FM][FN]) {
    NoSide none;
    parts<RAGGED, false, true>(A, lda, W, ldw, rows_valid, cols_valid, K, stages, acc, none);
  }
  // body() carrying side work at the ends of its rounds of four slices:
  // side.issue(u) after round u's last loads, side.fold(u) after round u+1
  // (u < Side::NPASS).  The caller guarantees K / (NST * BK) >= NPASS + 2,
  // so the side work ends before the last round that loads.
  static constexpr bool side_fits(int K, int npass) { return K / (NST * BK) >= npass + 2; }
  // K values the slice schedule covers exactly (whole rounds of four slices)
  static constexpr bool k_fits(int64_t K) { return K > 0 && K % KSTEP == 0; }
  // the operand loads address A's TM rows and W's K rows through 2 GiB
  // buffer resources (32-bit offsets from the tile's origin)
  static constexpr bool operands_fit(int64_t lda, int64_t ldw, int64_t K) {
    return ((int64_t)TM * lda + K) * 2 < (int64_t(1) << 31) && K * ldw * 2 < (int64_t(1) << 31);
  }
  template <bool RAGGED, class Side>
  __device__ static __forceinline__ void body_side(const uint16_t* __restrict__ A, int64_t lda,
                                                   const uint16_t* __restrict__ W, int64_t ldw,
                                                   int rows_valid, int cols_valid, int K,
                                                   char* const (&stages)[4], floatx16 (&acc)[FM][FN],
                                                   Side& side) {
    parts<RAGGED, false, true>(A, lda, W, ldw, rows_valid, cols_valid, K, stages, acc, side);
  }

  template <bool RAGGED, bool PRO, bool BODY, class Side = NoSide>
  __device__ static __forceinline__ void parts(const uint16_t* __restrict__ A, int64_t lda,
                                               const uint16_t* __restrict__ W, int64_t ldw,
                                               int /*rows_valid*/, int /*cols_valid*/, int K,
                                               char* const (&stages)[4], floatx16 (&acc)[FM][FN],
                                               Side& side) {
    static_assert(!RAGGED, "full tiles only");
#if defined(__HIP_DEVICE_COMPILE__)
    const int tid = threadIdx.x, lane = opaque_lane(), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    if constexpr (BODY) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    }
    const int nk = K / BK;
    // precondition (every launcher checks k_fits(K)): K is a multiple of
    // NST * BK; otherwise nothing is loaded and the accumulators are NaN
    if (nk == 0 || nk % NST != 0 || K % BK != 0) {
      if constexpr (BODY) {
        if (K != 0) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_nanf("");
        }
      }
      return;
    }
    char* const a_st[2] = {direct_a_stage0(), direct_a_stage1()};

    const __amdgpu_buffer_rsrc_t rsa = raw_rsrc(A), rsw = raw_rsrc(W);
    uint32_t aoff[A_LD], woff[W_LD];
#pragma unroll
    for (int t = 0; t < A_LD; ++t) {
      const int b = t * NW + wave;
      const int row = b * AROWS_PER_BLOCK + lane / CA;
      const int c = (lane % CA) ^ ((row / (16 / CA)) % CA);
      aoff[t] = (uint32_t)(((int64_t)row * lda + c * 8) * 2);
    }
#pragma unroll
    for (int t = 0; t < W_LD; ++t) {
      const int b = t * NW + wave;
      const int k = b * WROWS_PER_BLOCK + lane / CW;
      const int c = (lane % CW) ^ (4 * (k & 3));
      woff[t] = (uint32_t)(((int64_t)k * ldw + c * 8) * 2);
    }
    // A rows [.., k0 .. k0+63] of double stage kd (k0 = 64 kd) into ab
    auto load_a = [&](char* ab, int kd) {
      const uint32_t ak = (uint32_t)kd * (2 * BK * 2);
#pragma unroll
      for (int t = 0; t < A_LD; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsa, (__attribute__((address_space(3))) void*)(ab + (t * NW + wave) * 1024), 16, aoff[t], ak, 0, 0);
    };
    auto load_w = [&](char* wb, int ks) {
      const uint32_t wk = (uint32_t)ks * (uint32_t)(BK * ldw * 2);
#pragma unroll
      for (int t = 0; t < W_LD; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsw, (__attribute__((address_space(3))) void*)(wb + (t * NW + wave) * 1024), 16, woff[t], wk, 0, 0);
    };

    typedef short short4v __attribute__((ext_vector_type(4)));
    // fragments of k-substep kk of a slice: its A rows from half h of double
    // stage ab, its W rows from stage wb
    auto read_frags = [&](const char* ab, int h, const char* wb, int kk, bf16x8 (&a)[FM], bf16x8 (&b)[FN]) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = wm * WTM + 32 * i + (lane & 31);
        const int c = (h * 4 + kk * 2 + (lane >> 5)) ^ ((m / (16 / CA)) % CA);
        a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ab + m * (2 * BK * 2) + c * 16));
      }
      const int G = lane >> 4, s = lane & 15;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * WTN + 32 * j + (G & 1) * 16 + 4 * (s & 3);
        short4v hv[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int k = kk * 16 + (G >> 1) * 8 + 4 * hh + (s >> 2);
          const int c = (n >> 3) ^ (4 * (k & 3));
          const char* p = wb + k * (TN * 2) + c * 16 + (n & 7) * 2;
          hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
        }
        const short __attribute__((ext_vector_type(8))) v8 = {hv[0][0], hv[0][1], hv[0][2], hv[0][3],
                                                             hv[1][0], hv[1][1], hv[1][2], hv[1][3]};
        b[j] = __builtin_bit_cast(bf16x8, v8);
      }
    };
    auto mfmas = [&](const bf16x8 (&a)[FM], const bf16x8 (&b)[FN]) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    };
    constexpr int ND = FM + 2 * FN;
    constexpr int NM = FM * FN;
    bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];

    auto sync_n = [&](auto n_c) {
      constexpr int N = decltype(n_c)::value;
      static_assert(N <= 63, "vmcnt range");
      __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);  // vmcnt(N) lgkmcnt(0)
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    };
    // slice j = j0 + S of a round (W stage S, A double stage S / 2, half S % 2);
    // LOAD: issue W(j+4) and, for odd S, A(j+3 .. j+4); NEXT: read slice j+1's
    // first fragments; N: this slice's wait count
    auto slice = [&](auto s_c, auto load_c, auto next_c, auto n_c, int j) {
      constexpr int S = decltype(s_c)::value;
      char* const wb = stages[S];
      char* const ab = a_st[S / 2];
      read_frags(ab, S % 2, wb, 1, fa1, fb1);
      mfmas(fa0, fb0);
      interleave<NM, ND, 0>();
      sync_n(n_c);
      constexpr bool LOADA = decltype(load_c)::value && (S % 2 == 1);
      if constexpr (decltype(load_c)::value) load_w(wb, j + NST);
      if constexpr (LOADA) load_a(a_st[((S + 3) / 2) % 2], (j + 3) / 2);
      if constexpr (decltype(next_c)::value)
        read_frags(a_st[((S + 1) % NST) / 2], (S + 1) % 2, stages[(S + 1) % NST], 0, fa0, fb0);
      mfmas(fa1, fb1);
      interleave<NM, decltype(next_c)::value ? ND : 0,
                 decltype(load_c)::value ? W_LD + (LOADA ? A_LD : 0) : 0>();
    };
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;

    if constexpr (PRO) {
      load_a(a_st[0], 0);
      load_w(stages[0], 0);
      load_w(stages[1], 1);
      load_a(a_st[1], 1);
      load_w(stages[2], 2);
    }
    if constexpr (!BODY) return;
    load_w(stages[3], 3);
    sync_n(std::integral_constant<int, 2 * W_LD + A_LD + W_LD>{});  // slice 0 landed: W(1), A(2..3), W(2), W(3) may not have
    read_frags(a_st[0], 0, stages[0], 0, fa0, fb0);

    auto round = [&](auto pv_c, auto loads_c, int j0) {
      constexpr int PV = decltype(pv_c)::value;
      using L_ = decltype(loads_c);
      if constexpr (L_::value) {
        slice(std::integral_constant<int, 0>{}, T_{}, T_{}, std::integral_constant<int, 2 * W_LD + A_LD + PV>{}, j0);
        slice(std::integral_constant<int, 1>{}, T_{}, T_{}, std::integral_constant<int, W_LD + PV>{}, j0 + 1);
        slice(std::integral_constant<int, 2>{}, T_{}, T_{}, std::integral_constant<int, 2 * W_LD + A_LD + PV>{}, j0 + 2);
        slice(std::integral_constant<int, 3>{}, T_{}, T_{}, std::integral_constant<int, W_LD>{}, j0 + 3);
      } else {
        slice(std::integral_constant<int, 0>{}, F_{}, T_{}, std::integral_constant<int, 2 * W_LD + A_LD + PV>{}, j0);
        slice(std::integral_constant<int, 1>{}, F_{}, T_{}, std::integral_constant<int, 0>{}, j0 + 1);
        slice(std::integral_constant<int, 2>{}, F_{}, T_{}, std::integral_constant<int, 0>{}, j0 + 2);
        slice(std::integral_constant<int, 3>{}, F_{}, F_{}, std::integral_constant<int, 0>{}, j0 + 3);
      }
    };
    auto side_step = [&](auto fold_c, auto issue_c, int u) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(fold_c)::value) side.fold(u - 1);
      if constexpr (decltype(issue_c)::value) side.issue(u);
      __builtin_amdgcn_sched_barrier(0);
    };
    using Z_ = std::integral_constant<int, 0>;
    using PV_ = std::integral_constant<int, Side::V>;
    const int nr = nk / NST;
    int r = 0;
    if constexpr (Side::NPASS > 0) {
      round(Z_{}, T_{}, 0);
      side_step(F_{}, T_{}, 0);
      for (r = 1; r < Side::NPASS; ++r) {
        round(PV_{}, T_{}, r * NST);
        side_step(T_{}, T_{}, r);
      }
      round(PV_{}, T_{}, r * NST);
      side_step(T_{}, F_{}, r);
      ++r;
    }
    for (; r < nr - 1; ++r) round(Z_{}, T_{}, r * NST);
    round(Z_{}, F_{}, (nr - 1) * NST);
#endif
  }
};

template <int TM_, int TN_, int WM_, int WN_>
struct TileF32 {
  static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
  static constexpr bool kSplitMainloop = false;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int BK = 32;
  static constexpr int LDA = BK + 1, LDB = TN + 4;
  static constexpr int WTM = TM / WM, WTN = TN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_ELEMS = TM * LDA, B_ELEMS = BK * LDB, STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * 4;
  static constexpr int SMEM_BYTES = LDS_BYTES;  // stage array 0 holds everything
  static constexpr int NST = 1;
  static constexpr int A_LD = (TM * BK / 4) / NT, B_LD = (BK * TN / 4) / NT;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(A_LD >= 1 && B_LD >= 1 && (TM * BK / 4) % NT == 0 && (BK * TN / 4) % NT == 0,
                "slices must split evenly");

  // Tile coordinates of accumulator elements acc[i][j][4g .. 4g+3]: one row, 4 columns.
  __device__ static __forceinline__ void quad(int i, int j, int g, int lane, int wave, int& row,
                                              int& col0) {
    const int wm = wave / WN, wn = wave % WN;
    row = wm * WTM + 32 * i + (lane & 31);
    col0 = wn * WTN + 32 * j + 8 * g + 4 * (lane >> 5);
  }

  // Stores the accumulators of this lane into a row-major tile at `base`
  // (leading dimension ld, element type DT): one base pointer per lane, the
  // block and group offsets are compile-time constants.
  template <int DT, bool RAGGED>
  __device__ static __forceinline__ void store_acc(void* base, int64_t ld, int rows_valid,
                                                   int cols_valid, const floatx16 (&acc)[FM][FN]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = (wave / WN) * WTM + (lane & 31);
    const int c0 = (wave % WN) * WTN + 4 * (lane >> 5);
    constexpr int ES = DT == kBF16 ? 2 : 4;
    char* p = reinterpret_cast<char*>(base) + ((int64_t)r0 * ld + c0) * ES;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      char* pi = p + (int64_t)(32 * i) * ld * ES;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (RAGGED && (r0 + 32 * i >= rows_valid || c0 + 32 * j + 8 * g >= cols_valid)) continue;
          const floatx4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                             acc[i][j][4 * g + 3]};
          st4<DT>(pi + (32 * j + 8 * g) * ES, 0, v);
        }
      // keep the scheduler from hoisting every block's conversion at once
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  template <bool RAGGED>
  __device__ static __forceinline__ void run(const float* __restrict__ A, int64_t lda,
                                             const float* __restrict__ W, int64_t ldw,
                                             int rows_valid, int cols_valid, int K,
                                             char* const (&stages)[4], floatx16 (&acc)[FM][FN]) {
    float* const lds = reinterpret_cast<float*>(stages[0]);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // (vector types, not the float4 struct: an aggregate copy of the struct
    // into LDS kept these staging registers on the stack)
    // A ring of D slices in registers: slice ks + D is requested while slice
    // ks is computed, so D slices' load latencies overlap (the small-K calls
    // this tile serves are bound by that latency, not by the matrix cores).
    constexpr int D = 8;
    floatx4 ra[D][A_LD], rb[D][B_LD];
    const int nk = (K + BK - 1) / BK;

    auto load_global = [&](int ks, floatx4 (&pa)[A_LD], floatx4 (&pb)[B_LD]) {
      const int k0 = ks * BK;
#pragma unroll
      for (int t = 0; t < A_LD; ++t) {
        const int c = tid + t * NT;
        const int row = c / (BK / 4), k = k0 + (c % (BK / 4)) * 4;
        if (!RAGGED || (row < rows_valid && k < K))
          pa[t] = *reinterpret_cast<const floatx4*>(A + (int64_t)row * lda + k);
        else
          pa[t] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int t = 0; t < B_LD; ++t) {
        const int c = tid + t * NT;
        const int k = k0 + c / (TN / 4), n = (c % (TN / 4)) * 4;
        if (!RAGGED || (k < K && n < cols_valid))
          pb[t] = *reinterpret_cast<const floatx4*>(W + (int64_t)k * ldw + n);
        else
          pb[t] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    };
    auto store_lds = [&](int stage, const floatx4 (&pa)[A_LD], const floatx4 (&pb)[B_LD]) {
      float* As = lds + stage * STAGE;
      float* Bs = As + A_ELEMS;
#pragma unroll
      for (int t = 0; t < A_LD; ++t) {
        const int c = tid + t * NT;
        const int row = c / (BK / 4), kq = (c % (BK / 4)) * 4;
        As[row * LDA + kq + 0] = pa[t][0];
        As[row * LDA + kq + 1] = pa[t][1];
        As[row * LDA + kq + 2] = pa[t][2];
        As[row * LDA + kq + 3] = pa[t][3];
      }
#pragma unroll
      for (int t = 0; t < B_LD; ++t) {
        const int c = tid + t * NT;
        const int k = c / (TN / 4), n = (c % (TN / 4)) * 4;
        *reinterpret_cast<floatx4*>(Bs + k * LDB + n) = pb[t];
      }
    };
    auto compute = [&](int stage) {
      const float* As = lds + stage * STAGE;
      const float* Bs = As + A_ELEMS;
#pragma unroll
      for (int kk = 0; kk < BK / 2; ++kk) {
        const int k = kk * 2 + (lane >> 5);
        float a[FM], b[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = As[(wm * WTM + 32 * i + (lane & 31)) * LDA + k];
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = Bs[k * LDB + wn * WTN + 32 * j + (lane & 31)];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(b[j], a[i], acc[i][j], 0, 0, 0);
      }
    };

    if (nk == 0) return;
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < nk) load_global(d, ra[d], rb[d]);
    store_lds(0, ra[0], rb[0]);
    __syncthreads();
    for (int ks0 = 0; ks0 < nk; ks0 += D) {
      // ring slot u holds slice ks0 + u until it is in LDS, then slice ks0 + u + D
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int ks = ks0 + u;
        if (ks < nk) {
          if (ks + D < nk) load_global(ks + D, ra[u], rb[u]);
          compute(ks & 1);
          if (ks + 1 < nk) store_lds((ks + 1) & 1, ra[(u + 1) % D], rb[(u + 1) % D]);
          __syncthreads();
        }
      }
    }
  }
};

}  // namespace hocf
