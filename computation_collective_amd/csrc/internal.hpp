// Launch-side declarations shared by the C ABI (abi.cpp) and the kernel
// translation units.  Arguments reaching these functions are validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace hocf {

struct GemmRsArgs {
  const void* A;
  const void* W;
  // the reduced chunks go to every one of outs[0 .. nout): one output
  // [M][N] for a ReduceScatter, the P receive windows for an AllReduce
  void* outs[kMaxP];
  int nout;
  int mode;  // 0: fused ReduceScatter (nout == 1); 1: fused AllReduce (nout == P);
             // 2: unfused ReduceScatter (a GEMM kernel, then a fold kernel; nout == 1)
  void* win_data[kMaxP];
  uint32_t* win_flags[kMaxP];
  uint32_t* ws;
  int P, M, N, K, Mc;
  int slot_dt, out_dt;
  int mtiles, ntiles;  // tile grid of one chunk
  int64_t total;       // P (sources) * P (chunks) * mtiles * ntiles
  SyncArgs sync;
  uint64_t* trace;     // the trace build's per-iteration records (trace.hpp), else NULL
  int Nc;              // columns computed (N for a whole call; a column piece's width otherwise:
                       // W, the windows and the outputs then point at the piece's first column,
                       // N stays their leading dimension)
  int max_wg;          // cap on the persistent grid (0: none)
  // the unfused form only: when set, the fold kernel goes to fold_stream,
  // after a wait on gemm_done (recorded on the call's stream after the GEMM)
  void* fold_stream;
  void* gemm_done;
};

struct GemvArArgs {
  const uint16_t* x;
  const uint16_t* W;
  void* part;
  uint32_t* part_flags;
  void* win_data[kMaxP];
  uint32_t* win_flags[kMaxP];
  uint32_t* ws;
  int P, Mb, N, K, tile_n, ntiles;
  int slot_dt, out_dt;
  int64_t total;  // P * ntiles
  bool fused;     // false: the unfused baseline (a GEMV kernel, then a fold kernel)
  SyncArgs sync;
};

struct AgGemmArgs {
  const uint16_t* A;
  const uint32_t* chunk_flags;
  const uint16_t* W;
  void* out;
  uint32_t* ws;
  int P, Mc, N, K, out_dt;
  int mtiles, ntiles;
  SyncArgs sync;
};

struct EmbbagArgs {
  const float* tables;
  const int32_t* indices;
  const int64_t* offsets;
  float* win_data[kMaxP];
  uint32_t* win_flags[kMaxP];
  uint32_t* ws;
  int64_t R;
  int T, D, B, L, P, Bd, tile_bags, nj;
  int64_t total;  // T * P * nj
  SyncArgs sync;
};

constexpr int kMaxExperts = 64;  // local experts of one GEMM + All-to-All call

struct GemmA2aArgs {
  const uint16_t* X;     // [T][K] token rows, grouped by expert
  const uint16_t* W;     // [E][K][N]
  const int32_t* dest;   // [T] destination rank of each row (-1: padding)
  const int32_t* slot;   // [T] row of the destination's window
  void* win_data[kMaxP];       // [cap][N] out_dt each
  uint32_t* win_flags[kMaxP];  // [1] each
  uint32_t expected[kMaxP];    // pieces (row x column tile) each destination receives
  int64_t row_off[kMaxExperts + 1];  // expert row ranges (whole row tiles)
  int tile_off[kMaxExperts + 1];     // first work item of each expert
  uint32_t* ws;
  int64_t T, cap;
  int P, E, N, K, ntiles, out_dt;
  int total;  // tiles: row tiles x column tiles over all experts
  int keep;   // tiles [0, keep) run whole; each later tile runs as `split` tiles of
  int split;  // tile_m / split rows (split = 1, 2 or 4; keep == total when 1)
  SyncArgs sync;
};

// All-to-All + GEMM (the MoE dispatch): router entries are taken in chunks
// of kA2gChunk of one source rank.
constexpr int kA2gChunk = 256;

struct A2aGemmArgs {
  const uint16_t* X;        // [P][B][K] token rows of the source ranks
  const int32_t* experts;   // [P][B][topk] global expert ids
  const uint16_t* W;        // [E][K][N]
  uint16_t* recv;           // [cap][K] received rows, grouped by local expert
  void* Y;                  // [cap][N] out_dt
  int64_t* expert_offsets;  // [E+1]
  int32_t* dest;            // [cap]
  int32_t* slot;            // [cap]
  int64_t* send_counts;     // [P]
  // workspace (uint32): misc words [0] delivery claim counter, [1] nonzero
  // when the rows exceed cap, [2] expert tiles, [3] spare, [4..12) the tile
  // queues' claim counters (one per XCD); per chunk a histogram and its
  // exclusive scan ([C][E+1]: local experts, then pairs landing here from
  // the chunk); per expert the group's first row [E+1], its pairs [E], its
  // first tile [E+1]; per row tile the rows that have landed [nrt]
  uint32_t *misc, *hist, *base, *grp, *cnt, *toff, *arrivals;
  int64_t cap;
  int P, E, e0, B, topk, N, K, out_dt, tile_m, ntiles, C, cps, nrt;
  int64_t max_tiles;  // tiles the grid is sized for: (cap / tile_m) * ntiles
  SyncArgs sync;
};

// Device properties the launches need, cached per device.
struct DeviceInfo {
  int cus = 0;
  int64_t wall_clock_khz = 0;
};
hipError_t device_info(DeviceInfo* out);

// Persistent-grid size for a kernel: resident workgroups the device can hold
// (occupancy x CUs), capped by the work available.
hipError_t persistent_grid(const void* kernel, int threads, int64_t work, int* grid, int cap = 0);

// The decomposed GEMM + ReduceScatter: `pieces` (<= kMaxPieces) column pieces, each an
// unfused GEMM (grid capped to leave `fold_cus` CUs) on s, then its fold on
// coll after an event; s waits for coll's last fold.
int launch_gemm_rs_pieces(const GemmRsArgs& a, int tile_m, int tile_n, int in_dt, int pieces, int fold_cus,
                          hipStream_t s, hipStream_t coll);

// Each returns hipSuccess, the HIP error a runtime call gave (a hipError_t
// value), or kNoKernel when it has no kernel for the shape (found before
// anything is enqueued).
constexpr int kNoKernel = -1;
constexpr int kMaxPieces = 16;  // column pieces of the decomposed GEMM + ReduceScatter
int launch_gemm_rs(const GemmRsArgs& a, int tile_m, int tile_n, int in_dt, hipStream_t s);
int launch_gemv_ar(const GemvArArgs& a, hipStream_t s);
int launch_ag_gemm(const AgGemmArgs& a, int tile_m, int tile_n, hipStream_t s);
int launch_embbag_a2a(const EmbbagArgs& a, hipStream_t s);
int launch_gemm_a2a(const GemmA2aArgs& a, int tile_m, hipStream_t s);
int launch_a2a_gemm(const A2aGemmArgs& a, bool fused, hipStream_t s);

// Workspace words each operator needs.
constexpr int64_t kWsBaseWords = kNumQueues + 1;

// The entry point that allocates nothing: the size of its per-device
// scratch (HOCF_NOALLOC_SCRATCH_BYTES), the device address of the current
// device's copy, and a kernel that zeroes n words of it on a stream.
constexpr int64_t kNoAllocScratchBytes = int64_t(1) << 20;
hipError_t noalloc_scratch(void** out);
int launch_zero_words(uint32_t* p, int64_t n, hipStream_t s);

}  // namespace hocf
