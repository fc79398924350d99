// Tile publication into receive windows, and the fixed-order reduction of
// published tiles, with device-coherent memory accesses.
//
// MI355X has one L2 per XCD, and the L2s are not coherent with each other
// for ordinary (write-back) accesses.  A fence at device scope therefore
// writes back every dirty line of the issuing XCD's L2 (release) or
// invalidates all of it (acquire) -- an L2-wide operation that stalls the
// issuing workgroup and, for an invalidate, evicts the A/W panels that every
// other workgroup on that XCD is streaming.  At one release per 256x256
// tile that costs more than the tile's stores.
//
// Published data never needs those fences if every access to it is itself
// coherent at device scope: the stores below carry the SC1 cache-policy bit
// (the policy the compiler gives device-scope atomic stores: written
// through to the memory side), and the reducer's loads carry SC1 as well
// (device-scope atomic loads: never served from a possibly stale line).
// Both also carry NT, the streaming hint: coherence is the SC bits' business,
// NT only keeps this use-once traffic from evicting the operand panels.
// The ordering a flag needs is then only that the data stores have
// completed before the flag store is issued -- an s_waitcnt vmcnt(0) in
// each thread and a barrier -- and, on the consumer side, that its data
// loads are issued after the flag (or arrival count) was seen.
//
// Write-through stores of partial lines are slow (each becomes its own
// memory-side write), while the MFMA accumulator layout gives every lane
// 16-byte pieces of 32 different rows.  So each wave first stages one
// 32-row block of its sub-tile in a wave-private LDS area, then stores it
// back row by row: a wave's store instruction covers 1 KB of contiguous
// row memory (whole 128-byte lines).
#pragma once

#include "common.hpp"

namespace hocf {

// Cache-policy operands: SC1 (device scope) with NT (streaming: published
// data is written once and read once, so it should not displace the GEMM
// operands in the caches), and none (ordinary write-back).
constexpr int kPolicyDevice = 16 | 2;
constexpr int kPolicyPlain = 0;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));


// 16-byte device-coherent accesses at byte offset voff (per lane) + soff
// (wave-uniform) from the resource's base.
template <int POLICY = kPolicyDevice>
__device__ __forceinline__ void st_dev16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                         u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, POLICY);
}
__device__ __forceinline__ u32x4 ld_dev16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kPolicyDevice);
}

// s_waitcnt vmcnt(0): every load and store this wave issued has completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// accesses (lgkmcnt(0)) but not for its global loads, which stay in flight.
// (__syncthreads() would also drain those.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Staging geometry of one wave's 32-row accumulator block.
template <class Tile, int DT>
struct PublishLayout {
  static constexpr int ES = DT == kBF16 ? 2 : 4;
  static constexpr int RB = Tile::WTN * ES;   // bytes per staged row
  static constexpr int NCH = RB / 16;         // 16-byte chunks per row
  static constexpr int WAVE_BYTES = 32 * RB;  // LDS per wave
  static_assert(NCH >= 2 && (NCH & (NCH - 1)) == 0, "row of a power-of-two number of chunks");
  static_assert(Tile::SMEM_BYTES % WAVE_BYTES == 0 || Tile::NW * WAVE_BYTES <= Tile::SMEM_BYTES,
                "a wave's staging area must not straddle two stage arrays");
  static_assert(Tile::NW * WAVE_BYTES <= (Tile::NST > 1 ? Tile::NST : 1) * Tile::SMEM_BYTES,
                "staging areas must fit in the stage arrays");

  __device__ static __forceinline__ char* area(char* const (&stages)[4], int wave) {
    const int off = wave * WAVE_BYTES;
    if constexpr (Tile::NW * WAVE_BYTES <= Tile::SMEM_BYTES) return stages[0] + off;
    else {
      // select without indexing the array at run time (it would have to live in memory)
      const int st = off / Tile::SMEM_BYTES;
      char* b = st == 0 ? stages[0] : st == 1 ? stages[1] : st == 2 ? stages[2] : stages[3];
      return b + off % Tile::SMEM_BYTES;
    }
  }
  // byte offset of 16-byte chunk c of staged row r (chunks XOR-swizzled by row)
  __device__ static __forceinline__ int at(int r, int c) { return r * RB + ((c ^ (r & (NCH - 1))) << 4); }
};

// Stores this workgroup's accumulators (a Tile-shaped tile) row-major at
// `dst` (leading dimension `ld` elements of type DT; wave-uniform) with the
// given cache policy, and (WAIT) waits until they have completed.  Uses the
// Tile's LDS stage arrays as staging space (begins with a barrier, so the
// mainloop's last reads are done).  Ragged tiles store only rows <
// rows_valid and columns < cols_valid (cols_valid a multiple of 16/ES).
// The caller's tile must satisfy TM * ld * ES < 2^31.
template <class Tile, int DT, bool RAGGED, int POLICY, bool WAIT>
__device__ __forceinline__ void store_tile(char* dst, int64_t ld, int rows_valid, int cols_valid,
                                           const floatx16 (&acc)[Tile::FM][Tile::FN],
                                           char* const (&stages)[4]) {
  using L = PublishLayout<Tile, DT>;
  constexpr int RPI = 64 / L::NCH;       // staged rows per store instruction
  constexpr int NIT = L::NCH / 2;        // store instructions per 32-row block
  constexpr int BATCH = NIT < 8 ? NIT : 8;
  const int wave = threadIdx.x >> 6;
  const int lane = opaque_lane();
  const int wm = wave / Tile::WN, wn = wave % Tile::WN;
  const int lr = lane & 31, half = lane >> 5;
  const int sr = lane / L::NCH, sc = lane % L::NCH;  // staged row / chunk this lane stores
  const __amdgpu_buffer_rsrc_t rs = raw_rsrc(dst);
  // this lane's store offset within the wave's first row block; rows move via soffset
  const uint32_t voff = (uint32_t)(((int64_t)(wm * Tile::WTM + sr) * ld + wn * Tile::WTN +
                                    sc * (16 / L::ES)) * L::ES);
  const int tcol = wn * Tile::WTN + sc * (16 / L::ES);
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
        if constexpr (DT == kBF16) {
          u32x2 u = {pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                     pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
          *reinterpret_cast<u32x2*>(p) = u;
        } else {
          const floatx4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                             acc[i][j][4 * g + 3]};
          *reinterpret_cast<floatx4*>(p) = v;
        }
      }
    // staged rows -> memory, 64 chunks (two to eight rows) per instruction;
    // LDS operations of one wave complete in order, so no barrier is needed
    // (the clobber: lanes read rows other lanes wrote, so the compiler must
    // not reuse loads from the previous block)
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int it0 = 0; it0 < NIT; it0 += BATCH) {
      u32x4 v[BATCH];
#pragma unroll
      for (int b = 0; b < BATCH; ++b)
        v[b] = *reinterpret_cast<const u32x4*>(area + L::at((it0 + b) * RPI + sr, sc));
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int rb = 32 * i + (it0 + b) * RPI;  // row of lane group 0, relative to wm * WTM
        const int trow = wm * Tile::WTM + rb + sr;
        if (!RAGGED || (trow < rows_valid && tcol < cols_valid))
          st_dev16<POLICY>(rs, voff, (uint32_t)((int64_t)rb * ld * L::ES), v[b]);
      }
    }
  }
  if constexpr (WAIT) wait_memory();
}

// Publication of a tile: device-coherent stores, complete when this returns.
template <class Tile, int DT, bool RAGGED>
__device__ __forceinline__ void publish_tile(char* dst, int64_t ld, int rows_valid, int cols_valid,
                                             const floatx16 (&acc)[Tile::FM][Tile::FN],
                                             char* const (&stages)[4]) {
  store_tile<Tile, DT, RAGGED, kPolicyDevice, true>(dst, ld, rows_valid, cols_valid, acc, stages);
}

// Where a reduced band goes: the same bytes at byte offset `off` from each
// of the `n` output bases -- one for a ReduceScatter (the destination's
// chunk), all P receive windows for an AllReduce.  `base` points at the
// kernel's argument array, so the addresses are wave-uniform.
struct OutSet {
  void* const* base;
  int n;
  int64_t off;
  __device__ __forceinline__ char* at(int d) const { return reinterpret_cast<char*>(base[d]) + off; }
};

// Geometry of the fixed-order reduction of one Tile with slot type SDT:
// 16-byte chunks, CPR per tile row, RPS rows per pass of the workgroup, and
// the pieces a tile's reduction is cut into (at least 32 rows or one pass).
template <class Tile, int SDT>
struct ReduceLayout {
  static constexpr int SES = SDT == kBF16 ? 2 : 4;
  static constexpr int CE = 16 / SES;              // elements per 16-byte chunk
  static constexpr int CPR = Tile::TN / CE;        // chunks per tile row
  static constexpr int RPS = Tile::NT / CPR;       // rows covered by one pass of the workgroup
  static constexpr int PIECE_ROWS = RPS > Tile::TM / 8 ? RPS : Tile::TM / 8;
  static constexpr int PIECES = Tile::TM / PIECE_ROWS;
  static_assert(Tile::NT % CPR == 0 && PIECE_ROWS % RPS == 0 && Tile::TM % PIECE_ROWS == 0,
                "reduce layout");
};

// Fixed-order reduction of rows [row0, row0 + PIECE_ROWS) of one published
// tile: for every element, acc = slot 0; acc += slot q for q = 1 .. P-1
// (fp32, in rank order); the result is rounded to ODT and stored at `out`
// (the output tile's origin, leading dimension ld_out).  Slot q's tile starts
// at slot0 + q * slot_bytes (leading dimension ld, element type SDT); all
// pointers are wave-uniform.  Loads are device-coherent; U chunks of 16
// bytes per thread and slot (PMAX slots, those past P re-reading slot P-1)
// are in flight together.  Requires P <= PMAX and TM * ld * ES(SDT) < 2^31.
template <class Tile, int SDT, int ODT, bool RAGGED, int PMAX, int U>
__device__ __forceinline__ void reduce_piece(const char* slot0, int64_t slot_bytes, int P, int64_t ld,
                                             const OutSet& outs, int64_t ld_out, int row0, int rows_valid,
                                             int cols_valid) {
  using L = ReduceLayout<Tile, SDT>;
  constexpr int SES = L::SES, CE = L::CE, CPR = L::CPR, RPS = L::RPS;
  constexpr int NPASS = L::PIECE_ROWS / RPS;
  constexpr int UE = U < NPASS ? U : NPASS;
  static_assert(NPASS % UE == 0, "reduce layout");
  const int tid = (int)(threadIdx.x & ~63) + opaque_lane();
  const int r0 = row0 + tid / CPR, col = (tid % CPR) * CE;
  const uint32_t voff = (uint32_t)(((int64_t)r0 * ld + col) * SES);
  const int64_t orel = ((int64_t)r0 * ld_out + col) * (ODT == kBF16 ? 2 : 4);
  for (int ps = 0; ps < NPASS; ps += UE) {
    u32x4 v[UE][PMAX];
#pragma unroll
    for (int q = 0; q < PMAX; ++q) {
      // slots beyond P re-read slot P-1 (loads stay unconditional); they are not added
      const int qq = q < P ? q : P - 1;
      const __amdgpu_buffer_rsrc_t rs = raw_rsrc(slot0 + qq * slot_bytes);
#pragma unroll
      for (int u = 0; u < UE; ++u) {
        if constexpr (RAGGED) {
          // rows and columns past the tile's edge read its last valid chunk (not stored)
          const int row = min((ps + u) * RPS + r0, rows_valid - 1);
          const int c = min(col, cols_valid - CE);
          v[u][q] = ld_dev16(rs, (uint32_t)(((int64_t)row * ld + c) * SES), 0);
        } else {
          v[u][q] = ld_dev16(rs, voff, (uint32_t)((int64_t)(ps + u) * RPS * ld * SES));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int row = (ps + u) * RPS + r0;
      if (RAGGED && (row >= rows_valid || col >= cols_valid)) continue;
      const int64_t o = orel + (int64_t)(ps + u) * RPS * ld_out * (ODT == kBF16 ? 2 : 4);
      if constexpr (SDT == kF32) {
        floatx4 s = __builtin_bit_cast(floatx4, v[u][0]);
#pragma unroll
        for (int q = 1; q < PMAX; ++q)
          if (q < P) s = s + __builtin_bit_cast(floatx4, v[u][q]);
        for (int d = 0; d < outs.n; ++d) st4<ODT>(outs.at(d) + o, 0, s);
      } else {
        floatx4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < PMAX; ++q) {
          const u32x4 w = v[u][q];
          const floatx4 a = {bf16_to_f32(w[0] & 0xffffu), bf16_to_f32(w[0] >> 16),
                             bf16_to_f32(w[1] & 0xffffu), bf16_to_f32(w[1] >> 16)};
          const floatx4 b = {bf16_to_f32(w[2] & 0xffffu), bf16_to_f32(w[2] >> 16),
                             bf16_to_f32(w[3] & 0xffffu), bf16_to_f32(w[3] >> 16)};
          if (q == 0) { lo = a; hi = b; }
          else if (q < P) { lo = lo + a; hi = hi + b; }
        }
        for (int d = 0; d < outs.n; ++d) {
          st4<ODT>(outs.at(d) + o, 0, lo);
          st4<ODT>(outs.at(d) + o, 4, hi);
        }
      }
    }
  }
}

// The fold of reduce_piece, for one band carried through a GEMM mainloop as
// its side work (TileBf16Direct::body_side): unit u is row pass u of the
// band, its PMAX device-coherent slot loads issued at the end of one K round
// and folded (rank order, fp32, rounded once to ODT) at the end of the next,
// so the loads' latency hides behind MFMA work.  Folded rows are parked in
// LDS (the mainloop may issue no vector-memory stores of its own) and
// written out by flush().  Same arithmetic and element order as
// reduce_piece; requires P <= PMAX and a window below 2 GiB from the
// band's slot 0 (P * slot_bytes < 2^31).
template <class Tile, int SDT, int ODT, int PMAX>
struct BandFold {
  using L = ReduceLayout<Tile, SDT>;
  static constexpr int NPASS = L::PIECE_ROWS / L::RPS;
  static constexpr int V = PMAX;
  static constexpr int OES = ODT == kBF16 ? 2 : 4;
  static constexpr int OUT_BYTES = L::CE * OES;  // one thread's result of one pass
  static constexpr int LDS_BYTES = NPASS * Tile::NT * OUT_BYTES;
  typedef __attribute__((address_space(3))) char lds_char;

  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff, slot_bytes, pass_bytes;
  int P;
  lds_char* park;
  u32x4 v[PMAX];

  // slot0: the band's tile in slot 0 (wave-uniform); area: LDS_BYTES of LDS
  __device__ __forceinline__ void init(const char* slot0, uint32_t slot_bytes_, int P_, int64_t ld, int row0,
                                       lds_char* area) {
    const int tid = (int)(threadIdx.x & ~63) + opaque_lane();
    const int r0 = row0 + tid / L::CPR, col = (tid % L::CPR) * L::CE;
    rs = raw_rsrc(slot0);
    voff = (uint32_t)(((int64_t)r0 * ld + col) * L::SES);
    slot_bytes = slot_bytes_;
    pass_bytes = (uint32_t)(L::RPS * ld * L::SES);
    P = P_;
    park = area + tid * OUT_BYTES;
  }
  __device__ __forceinline__ void issue(int pass) {
#pragma unroll
    for (int q = 0; q < PMAX; ++q) {
      const int qq = q < P ? q : P - 1;  // past P: re-read slot P-1, never added
      v[q] = ld_dev16(rs, voff, (uint32_t)qq * slot_bytes + (uint32_t)pass * pass_bytes);
    }
  }
  __device__ __forceinline__ void fold(int pass) {
    lds_char* o = park + pass * (Tile::NT * OUT_BYTES);
    if constexpr (SDT == kF32) {
      floatx4 s = __builtin_bit_cast(floatx4, v[0]);
#pragma unroll
      for (int q = 1; q < PMAX; ++q)
        if (q < P) s = s + __builtin_bit_cast(floatx4, v[q]);
      if constexpr (ODT == kBF16)
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(o) =
            u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
      else
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(o) = __builtin_bit_cast(u32x4, s);
    } else {
      floatx4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < PMAX; ++q) {
        const u32x4 w = v[q];
        const floatx4 a = {bf16_to_f32(w[0] & 0xffffu), bf16_to_f32(w[0] >> 16),
                           bf16_to_f32(w[1] & 0xffffu), bf16_to_f32(w[1] >> 16)};
        const floatx4 b = {bf16_to_f32(w[2] & 0xffffu), bf16_to_f32(w[2] >> 16),
                           bf16_to_f32(w[3] & 0xffffu), bf16_to_f32(w[3] >> 16)};
        if (q == 0) { lo = a; hi = b; }
        else if (q < P) { lo = lo + a; hi = hi + b; }
      }
      if constexpr (ODT == kBF16) {
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(o) =
            u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                  pack_bf16x2(hi[2], hi[3])};
      } else {
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(o) = __builtin_bit_cast(u32x4, lo);
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(o + 16) = __builtin_bit_cast(u32x4, hi);
      }
    }
  }
  // the parked rows -> every output of `outs` (the band's output tile
  // origins, leading dimension ld_out)
  __device__ __forceinline__ void flush(const OutSet& outs, int64_t ld_out, int row0) {
    const int tid = (int)(threadIdx.x & ~63) + opaque_lane();
    const int r0 = row0 + tid / L::CPR, col = (tid % L::CPR) * L::CE;
    const int64_t orel = ((int64_t)r0 * ld_out + col) * OES;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      const lds_char* src = park + pass * (Tile::NT * OUT_BYTES);
      const int64_t o = orel + (int64_t)pass * L::RPS * ld_out * OES;
      // (streaming stores: the folded rows are written once and not read
      // back by this kernel, so they should not displace operand panels)
      if constexpr (OUT_BYTES == 8) {
        const u32x2 w = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(src);
        for (int d = 0; d < outs.n; ++d) __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(outs.at(d) + o));
      } else {
        u32x4 w[OUT_BYTES / 16];
#pragma unroll
        for (int b = 0; b < OUT_BYTES / 16; ++b)
          w[b] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(src + 16 * b);
        for (int d = 0; d < outs.n; ++d)
#pragma unroll
          for (int b = 0; b < OUT_BYTES / 16; ++b)
            __builtin_nontemporal_store(w[b], reinterpret_cast<u32x4*>(outs.at(d) + o + 16 * b));
      }
    }
  }
};

}  // namespace hocf
