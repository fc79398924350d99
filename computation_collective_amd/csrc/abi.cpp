// C ABI of libhocf.so: argument validation, launch-argument packing, error
// reporting.  Every check runs before anything is enqueued, so an invalid
// call leaves the stream untouched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "../../include/hocf.h"
#include "internal.hpp"
#include "trace.hpp"

namespace {

thread_local char g_err[512] = "";

hocf_status fail(hocf_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

hocf_status ok() {
  g_err[0] = 0;
  return HOCF_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Checks on the sync block (no HIP call).  `need` = workspace bytes the call needs.
hocf_status check_sync(const hocf_sync* s, size_t need) {
  if (!s) return fail(HOCF_ERR_INVALID_ARG, "sync is NULL");
  if (s->epoch == 0) return fail(HOCF_ERR_INVALID_ARG, "epoch must be nonzero");
  if (need > 0) {
    if (!s->workspace) return fail(HOCF_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned16(s->workspace)) return fail(HOCF_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    if (s->workspace_bytes < need)
      return fail(HOCF_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes", s->workspace_bytes, need);
  }
  if (s->status && (reinterpret_cast<uintptr_t>(s->status) & 3u))
    return fail(HOCF_ERR_INVALID_ARG, "status word not 4-byte aligned");
  if (s->abort_flag && (reinterpret_cast<uintptr_t>(s->abort_flag) & 3u))
    return fail(HOCF_ERR_INVALID_ARG, "abort word not 4-byte aligned");
  return HOCF_OK;
}

// Converts a checked sync block for the kernels (queries the device clock).
hocf_status to_sync_args(const hocf_sync* s, hocf::SyncArgs* out) {
  hocf::DeviceInfo di;
  if (hocf::device_info(&di) != hipSuccess) return fail(HOCF_ERR_HIP, "device query failed");
  const uint64_t ns = s->spin_timeout_ns ? s->spin_timeout_ns : 1000000000ull;
  out->epoch = s->epoch;
  out->status = s->status;
  out->abort_flag = s->abort_flag;
  // wall_clock64() ticks at wall_clock_khz kHz
  const long double ticks = (long double)ns * (long double)di.wall_clock_khz / 1.0e6L;
  out->timeout_ticks = ticks > 1.8e19L ? ~0ull : (uint64_t)ticks;
  return HOCF_OK;
}

hocf_status check_windows(const hocf_window* win, int P, const char* what) {
  if (!win) return fail(HOCF_ERR_INVALID_ARG, "%s: window array is NULL", what);
  for (int r = 0; r < P; ++r) {
    if (!win[r].data || !win[r].flags)
      return fail(HOCF_ERR_INVALID_ARG, "%s: window %d has a NULL data or flags pointer", what, r);
    if (!aligned16(win[r].data) || (reinterpret_cast<uintptr_t>(win[r].flags) & 3u))
      return fail(HOCF_ERR_INVALID_ARG, "%s: window %d misaligned", what, r);
  }
  return HOCF_OK;
}

bool dt_ok(hocf_dtype d) { return d == HOCF_F32 || d == HOCF_BF16; }

// Byte ranges a call reads (inputs) and writes (outputs).  A written range
// may overlap no other range of the call: the kernels read their inputs
// while other workgroups already write, and publish into windows that others
// read, so any aliasing gives unspecified results.  Read-only ranges may
// overlap each other.  Empty ranges and NULL pointers are skipped.
class Ranges {
 public:
  void in(const char* what, int idx, const void* p, int64_t bytes) { add(what, idx, p, bytes, false); }
  void out(const char* what, int idx, const void* p, int64_t bytes) { add(what, idx, p, bytes, true); }
  hocf_status check(const char* op) const {
    for (int i = 0; i < n_; ++i)
      for (int j = i + 1; j < n_; ++j) {
        const R& a = r_[i];
        const R& b = r_[j];
        if (!a.out && !b.out) continue;
        if (a.lo < b.hi && b.lo < a.hi)
          return fail(HOCF_ERR_INVALID_ARG, "%s: %s[%d] and %s[%d] overlap (an output may alias nothing else)",
                      op, a.what, a.idx, b.what, b.idx);
      }
    return HOCF_OK;
  }

 private:
  struct R {
    const char* what;
    int idx;
    uintptr_t lo, hi;
    bool out;
  };
  void add(const char* what, int idx, const void* p, int64_t bytes, bool out) {
    if (!p || bytes <= 0 || n_ >= kMax) return;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    r_[n_++] = R{what, idx, lo, lo + (uintptr_t)bytes, out};
  }
  static constexpr int kMax = 4 * HOCF_MAX_P + 16;
  R r_[kMax];
  int n_ = 0;
};

// The sync block's own ranges: the status word and the workspace (both written).
void add_sync(Ranges& rg, const hocf_sync* s, size_t ws_bytes) {
  rg.out("status", 0, s->status, 4);
  rg.out("workspace", 0, s->workspace, (int64_t)ws_bytes);
}

hocf_status launched(int e, const char* what) {
  if (e == hocf::kNoKernel) return fail(HOCF_ERR_UNSUPPORTED, "%s: no kernel for this shape", what);
  if (e != hipSuccess) return fail(HOCF_ERR_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(e)));
  return ok();
}

}  // namespace

namespace hocf {

hipError_t device_info(DeviceInfo* out) {
  static std::mutex mu;
  static std::unordered_map<int, DeviceInfo> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    DeviceInfo di;
    int v = 0;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    di.cus = v;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return e;
    di.wall_clock_khz = v > 0 ? v : 100000;
    it = cache.emplace(dev, di).first;
  }
  *out = it->second;
  return hipSuccess;
}

hipError_t persistent_grid(const void* kernel, int threads, int64_t work, int* grid, int cap) {
  static std::mutex mu;
  static std::unordered_map<const void*, std::unordered_map<int, int>> occ;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  int per_cu = 0;
  {
    std::lock_guard<std::mutex> lk(mu);
    auto& m = occ[kernel];
    auto it = m.find(dev);
    if (it == m.end()) {
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
      if (e != hipSuccess) return e;
      if (per_cu < 1) per_cu = 1;
      m[dev] = per_cu;
    } else {
      per_cu = it->second;
    }
  }
  int64_t g = (int64_t)per_cu * di.cus;
  if (work < g) g = work;
  if (cap > 0 && cap < g) g = cap;
  // optional cap on the persistent grid (documented with the ABI)
  if (const char* cap = std::getenv("HOCF_MAX_WORKGROUPS")) {
    const long v = std::strtol(cap, nullptr, 10);
    if (v > 0 && v < g) g = v;
  }
  if (g < 1) g = 1;
  *grid = (int)g;
  return hipSuccess;
}

}  // namespace hocf

extern "C" {

int hocf_abi_version(void) { return HOCF_ABI_VERSION; }

const char* hocf_status_string(hocf_status s) {
  switch (s) {  // (any int: e.g. a status word read back from the device)
    case HOCF_OK: return "ok";
    case HOCF_ERR_INVALID_ARG: return "invalid argument";
    case HOCF_ERR_UNSUPPORTED: return "unsupported combination";
    case HOCF_ERR_HIP: return "HIP runtime error";
    case HOCF_ERR_TIMEOUT: return "flag wait timed out";
    case HOCF_ERR_ABORTED: return "aborted";
    case HOCF_ERR_BAD_INDEX: return "embedding index out of range";
    case HOCF_ERR_PROTOCOL: return "partial consumed before its flag was set";
    case HOCF_ERR_CAPACITY: return "more rows routed here than the receive buffer holds";
  }
  return "unknown status";
}

const char* hocf_last_error(void) { return g_err; }

/* ------------------------------------------------------------ GEMM + RS */

// The GEMM + ReduceScatter / AllReduce scheduler words, in bytes.
static size_t gemm_rs_sched_bytes(int P, int M, int N, int tile_m, int tile_n) {
  if (P <= 0 || M < 0 || N < 0 || tile_m <= 0 || tile_n <= 0 || M % P) return 0;
  const int64_t tpc = cdiv(M / P, tile_m) * cdiv(N, tile_n);
  // arrival counters [P][tpc], band queue heads and tails [8 + 8], band queues [8][P * tpc]
  return (size_t)(hocf::kWsBaseWords + (int64_t)P * tpc + 2 * hocf::kNumQueues +
                  (int64_t)hocf::kNumQueues * P * tpc) * 4;
}

// Where the trace build's per-iteration records start (after the scheduler words).
static size_t trace_offset(size_t sched) { return (sched + 255) & ~(size_t)255; }

size_t hocf_gemm_rs_workspace_bytes(int P, int M, int N, int tile_m, int tile_n) {
  const size_t sched = gemm_rs_sched_bytes(P, M, N, tile_m, tile_n);
  if (!hocf::kTraceBuild || sched == 0) return sched;
  return trace_offset(sched) + (size_t)hocf::kTraceBytes;
}

// Checks and launch shared by GEMM + ReduceScatter (one output) and GEMM +
// AllReduce (nout = P outputs, every one receiving all M rows).
// With noalloc, the scheduler words live in the library's per-device
// scratch instead of the caller's workspace (which must then be absent): it
// is zeroed on the stream before the kernel.
static hocf_status gemm_collective(const char* op, int P, int M, int N, int K, hocf_dtype in_dt,
                                   hocf_dtype slot_dt, hocf_dtype out_dt, const void* A, const void* W,
                                   const hocf_window* win, void* const* outs, int nout, int mode,
                                   int tile_m, int tile_n, const hocf_sync* sync, void* stream,
                                   bool noalloc = false, int pieces = 0, int fold_cus = 0,
                                   void* coll = nullptr) {
  if (P < 1 || P > HOCF_MAX_P) return fail(HOCF_ERR_INVALID_ARG, "%s: P=%d outside [1, %d]", op, P, HOCF_MAX_P);
  if (M < 0 || N < 0 || K < 0) return fail(HOCF_ERR_INVALID_ARG, "%s: negative dimension", op);
  if (M % P) return fail(HOCF_ERR_INVALID_ARG, "%s: M=%d not divisible by P=%d", op, M, P);
  if (!dt_ok(in_dt) || !dt_ok(slot_dt) || !dt_ok(out_dt))
    return fail(HOCF_ERR_INVALID_ARG, "%s: unknown dtype", op);
  const int vec = in_dt == HOCF_BF16 ? 8 : 4;
  if (N % vec || K % vec)
    return fail(HOCF_ERR_INVALID_ARG, "%s: N=%d and K=%d must be multiples of %d", op, N, K, vec);
  bool tile_ok;
  if (in_dt == HOCF_BF16) tile_ok = (tile_m == 256 && tile_n == 256) || (tile_m == 128 && tile_n == 128);
  else tile_ok = (tile_m == 64 && tile_n == 64) && slot_dt == HOCF_F32 && out_dt == HOCF_F32;
  if (!tile_ok)
    return fail(HOCF_ERR_UNSUPPORTED, "%s: no kernel for in=%d slot=%d out=%d tile %dx%d", op,
                in_dt, slot_dt, out_dt, tile_m, tile_n);
  // published tiles are addressed with 32-bit byte offsets from their origin
  if ((int64_t)tile_m * N * 4 >= ((int64_t)1 << 31))
    return fail(HOCF_ERR_UNSUPPORTED, "%s: tile_m * N = %lld elements per tile row band exceeds 2^29", op,
                (long long)tile_m * N);
  // (the no-allocation entry point holds the scheduler words only, never trace records)
  const size_t need = noalloc ? gemm_rs_sched_bytes(P, M, N, tile_m, tile_n)
                              : hocf_gemm_rs_workspace_bytes(P, M, N, tile_m, tile_n);
  hocf_status st;
  if (noalloc) {
    if (sync && (sync->workspace || sync->workspace_bytes))
      return fail(HOCF_ERR_INVALID_ARG, "%s: the workspace must be NULL (the library's scratch is used)", op);
    if (need > (size_t)hocf::kNoAllocScratchBytes)
      return fail(HOCF_ERR_UNSUPPORTED, "%s: %zu bytes of scheduler words exceed the %lld-byte scratch", op, need,
                  (long long)hocf::kNoAllocScratchBytes);
    st = check_sync(sync, 0);
  } else {
    st = check_sync(sync, need);
  }
  if (st != HOCF_OK) return st;
  if (M == 0 || N == 0) return ok();
  if (!A || !W || !outs) return fail(HOCF_ERR_INVALID_ARG, "%s: NULL tensor", op);
  if (K && (!aligned16(A) || !aligned16(W)))
    return fail(HOCF_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", op);
  const int64_t out_bytes = (int64_t)M * N * (out_dt == HOCF_BF16 ? 2 : 4);
  for (int q = 0; q < nout; ++q) {
    if (!outs[q]) return fail(HOCF_ERR_INVALID_ARG, "%s: NULL output %d", op, q);
    if (!aligned16(outs[q])) return fail(HOCF_ERR_INVALID_ARG, "%s: output %d not 16-byte aligned", op, q);
  }
  if ((st = check_windows(win, P, op)) != HOCF_OK) return st;
  {
    const int ies = in_dt == HOCF_BF16 ? 2 : 4, ses = slot_dt == HOCF_BF16 ? 2 : 4;
    const int64_t tpc = cdiv(M / P, tile_m) * cdiv(N, tile_n);
    Ranges rg;
    rg.in("A", 0, A, (int64_t)P * M * K * ies);
    rg.in("W", 0, W, (int64_t)P * K * N * ies);
    for (int q = 0; q < nout; ++q) rg.out("out", q, outs[q], out_bytes);
    for (int r = 0; r < P; ++r) {
      rg.out("win.data", r, win[r].data, (int64_t)M * N * ses);  // [P src][Mc][N]
      rg.out("win.flags", r, win[r].flags, (int64_t)P * tpc * 4);
    }
    add_sync(rg, sync, noalloc ? 0 : need);
    if ((st = rg.check(op)) != HOCF_OK) return st;
  }
  void* ws = sync->workspace;
  if (noalloc) {
    const hipError_t e = hocf::noalloc_scratch(&ws);
    if (e != hipSuccess) return fail(HOCF_ERR_HIP, "%s: scratch address: %s", op, hipGetErrorString(e));
  }

  hocf::SyncArgs sa;
  if ((st = to_sync_args(sync, &sa)) != HOCF_OK) return st;
  hocf::GemmRsArgs a{};
  a.A = A; a.W = W;
  for (int q = 0; q < nout; ++q) a.outs[q] = outs[q];
  a.nout = nout;
  a.mode = mode;
  for (int r = 0; r < P; ++r) { a.win_data[r] = win[r].data; a.win_flags[r] = win[r].flags; }
  a.ws = static_cast<uint32_t*>(ws);
  a.P = P; a.M = M; a.N = N; a.K = K; a.Mc = M / P;
  a.slot_dt = slot_dt; a.out_dt = out_dt;
  a.mtiles = (int)cdiv(a.Mc, tile_m);
  a.ntiles = (int)cdiv(N, tile_n);
  a.total = (int64_t)P * P * a.mtiles * a.ntiles;
  a.sync = sa;
  a.Nc = N;
  a.trace = nullptr;
  if (hocf::kTraceBuild && !noalloc)
    a.trace = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) +
                                          trace_offset(gemm_rs_sched_bytes(P, M, N, tile_m, tile_n)));
  if (noalloc) {
    const int e = hocf::launch_zero_words(a.ws, (int64_t)(need / 4), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return launched(e, op);
  }
  if (pieces > 0)
    return launched(hocf::launch_gemm_rs_pieces(a, tile_m, tile_n, in_dt, pieces, fold_cus,
                                                static_cast<hipStream_t>(stream), static_cast<hipStream_t>(coll)),
                    op);
  return launched(hocf::launch_gemm_rs(a, tile_m, tile_n, in_dt, static_cast<hipStream_t>(stream)), op);
}

hocf_status hocf_gemm_rs(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                         hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                         void* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream) {
  void* const outs[1] = {out};
  return gemm_collective("gemm_rs", P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, outs, 1, 0, tile_m, tile_n,
                         sync, stream);
}

hocf_status hocf_gemm_rs_unfused(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                                 hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                                 void* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream) {
  void* const outs[1] = {out};
  return gemm_collective("gemm_rs_unfused", P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, outs, 1, 2, tile_m,
                         tile_n, sync, stream);
}

hocf_status hocf_gemm_rs_noalloc(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                                 hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                                 void* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream) {
  void* const outs[1] = {out};
  return gemm_collective("gemm_rs_noalloc", P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, outs, 1, 0, tile_m,
                         tile_n, sync, stream, true);
}

hocf_status hocf_gemm_rs_decomposed(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                                    hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                                    void* out, int tile_m, int tile_n, int pieces, int fold_cus,
                                    const hocf_sync* sync, void* stream, void* coll_stream) {
  if (pieces < 1 || pieces > hocf::kMaxPieces)
    return fail(HOCF_ERR_INVALID_ARG, "gemm_rs_decomposed: pieces=%d outside [1, %d]", pieces, hocf::kMaxPieces);
  if (fold_cus < 0) return fail(HOCF_ERR_INVALID_ARG, "gemm_rs_decomposed: fold_cus=%d < 0", fold_cus);
  if (tile_n <= 0 || N % pieces || (N / pieces) % tile_n)
    return fail(HOCF_ERR_UNSUPPORTED, "gemm_rs_decomposed: N=%d is not %d pieces of whole %d-column tiles", N,
                pieces, tile_n);
  void* const outs[1] = {out};
  return gemm_collective("gemm_rs_decomposed", P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, outs, 1, 2, tile_m,
                         tile_n, sync, stream, false, pieces, fold_cus, coll_stream);
}

/* ------------------------------------------------------------ GEMM + AR */

size_t hocf_gemm_ar_workspace_bytes(int P, int M, int N, int tile_m, int tile_n) {
  return hocf_gemm_rs_workspace_bytes(P, M, N, tile_m, tile_n);
}

hocf_status hocf_gemm_ar(int P, int M, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                         hocf_dtype out_dt, const void* A, const void* W, const hocf_window* win,
                         void* const* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream) {
  return gemm_collective("gemm_ar", P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, out, P, 1, tile_m, tile_n,
                         sync, stream);
}

/* ------------------------------------------------------------ GEMM + A2A */

size_t hocf_gemm_a2a_workspace_bytes(int P) {
  if (P <= 0 || P > HOCF_MAX_P) return 0;
  return (size_t)(hocf::kWsBaseWords + P) * 4;
}

hocf_status hocf_gemm_a2a(int P, int E, int64_t T, int N, int K, hocf_dtype in_dt, hocf_dtype out_dt,
                          const void* X, const void* W, const int64_t* expert_offsets, const int32_t* dest,
                          const int32_t* slot, const int64_t* send_counts, const hocf_window* win, int64_t cap,
                          int tile_m, int tile_n, const hocf_sync* sync, void* stream) {
  if (P < 1 || P > HOCF_MAX_P) return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: P=%d outside [1, %d]", P, HOCF_MAX_P);
  if (E < 1 || E > hocf::kMaxExperts)
    return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: E=%d outside [1, %d]", E, hocf::kMaxExperts);
  if (T < 0 || N < 0 || K < 0 || cap < 0) return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: negative size");
  if (!dt_ok(in_dt) || !dt_ok(out_dt)) return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: unknown dtype");
  if (in_dt != HOCF_BF16) return fail(HOCF_ERR_UNSUPPORTED, "gemm_a2a: inputs must be bf16");
  if ((tile_m != 256 && tile_m != 128) || tile_n != 256)
    return fail(HOCF_ERR_UNSUPPORTED, "gemm_a2a: tile %dx%d (256x256 or 128x256 only)", tile_m, tile_n);
  if (tile_m == 128 && out_dt != HOCF_BF16)
    return fail(HOCF_ERR_UNSUPPORTED, "gemm_a2a: 128-row tiles take bf16 output only");
  if (N % 256 || K % 128)
    return fail(HOCF_ERR_UNSUPPORTED, "gemm_a2a: N=%d must be a multiple of 256 and K=%d of 128", N, K);
  if ((int64_t)K * N * 2 >= ((int64_t)1 << 31) || ((int64_t)tile_m * K + K) * 2 >= ((int64_t)1 << 31))
    return fail(HOCF_ERR_UNSUPPORTED, "gemm_a2a: an expert's W or a row tile exceeds 2 GiB");
  if (!expert_offsets || !send_counts) return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: NULL host array");
  if (expert_offsets[0] != 0 || expert_offsets[E] != T)
    return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: expert offsets must run from 0 to T=%lld", (long long)T);
  const int ntiles = N / tile_n;
  int64_t items = 0;
  for (int e = 0; e < E; ++e) {
    const int64_t n = expert_offsets[e + 1] - expert_offsets[e];
    if (n < 0 || n % tile_m)
      return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: expert %d has %lld rows (must be a non-negative multiple of %d)",
                  e, (long long)n, tile_m);
    items += n / tile_m * ntiles;
  }
  if (items >= ((int64_t)1 << 31)) return fail(HOCF_ERR_UNSUPPORTED, "gemm_a2a: too many tiles");
  for (int d = 0; d < P; ++d)
    if (send_counts[d] < 0 || send_counts[d] > cap || send_counts[d] * ntiles >= ((int64_t)1 << 32))
      return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: send_counts[%d]=%lld outside [0, cap=%lld]", d,
                  (long long)send_counts[d], (long long)cap);
  hocf_status st = check_sync(sync, hocf_gemm_a2a_workspace_bytes(P));
  if (st != HOCF_OK) return st;
  if ((st = check_windows(win, P, "gemm_a2a")) != HOCF_OK) return st;
  if (T > 0 && N > 0) {
    if (!X || !W || !dest || !slot) return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: NULL tensor");
    if (!aligned16(X) || !aligned16(W)) return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: tensors must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(dest) | reinterpret_cast<uintptr_t>(slot)) & 3u)
      return fail(HOCF_ERR_INVALID_ARG, "gemm_a2a: dest and slot must be 4-byte aligned");
  }
  {
    const int oes = out_dt == HOCF_BF16 ? 2 : 4;
    Ranges rg;
    rg.in("X", 0, X, T * K * 2);
    rg.in("W", 0, W, (int64_t)E * K * N * 2);
    rg.in("dest", 0, dest, T * 4);
    rg.in("slot", 0, slot, T * 4);
    for (int d = 0; d < P; ++d) {
      rg.out("win.data", d, win[d].data, cap * N * oes);
      rg.out("win.flags", d, win[d].flags, 4);
    }
    add_sync(rg, sync, hocf_gemm_a2a_workspace_bytes(P));
    if ((st = rg.check("gemm_a2a")) != HOCF_OK) return st;
  }

  hocf::SyncArgs sa;
  if ((st = to_sync_args(sync, &sa)) != HOCF_OK) return st;
  hocf::GemmA2aArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.W = static_cast<const uint16_t*>(W);
  a.dest = dest; a.slot = slot;
  for (int d = 0; d < P; ++d) {
    a.win_data[d] = win[d].data;
    a.win_flags[d] = win[d].flags;
    a.expected[d] = (uint32_t)(N > 0 ? send_counts[d] * ntiles : 0);
  }
  int64_t t = 0;
  for (int e = 0; e <= E; ++e) {
    a.row_off[e] = expert_offsets[e];
    a.tile_off[e] = (int)t;
    if (e < E) t += (expert_offsets[e + 1] - expert_offsets[e]) / tile_m * ntiles;
  }
  a.ws = static_cast<uint32_t*>(sync->workspace);
  a.T = T; a.cap = cap;
  a.P = P; a.E = E; a.N = N; a.K = K; a.ntiles = ntiles; a.out_dt = out_dt;
  a.total = (int)items;
  a.sync = sa;
  return launched(hocf::launch_gemm_a2a(a, tile_m, static_cast<hipStream_t>(stream)), "gemm_a2a");
}

/* ------------------------------------------------------------ A2A + GEMM */

// Router-entry chunks: kA2gChunk entries of one source each (at least one per source).
static int64_t a2g_chunks_per_source(int B, int topk) {
  const int64_t n = cdiv((int64_t)B * topk, hocf::kA2gChunk);
  return n > 0 ? n : 1;
}

size_t hocf_a2a_gemm_workspace_bytes(int P, int E, int B, int topk, int64_t cap, int tile_m) {
  if (P <= 0 || E <= 0 || B < 0 || topk < 0 || cap < 0 || tile_m <= 0) return 0;
  const int64_t C = (int64_t)P * a2g_chunks_per_source(B, topk);
  // misc [4 + 8 tile queues], hist and base [C][E+1] each, group rows [E+1], pairs [E], tiles [E+1],
  // arrivals [cap / tile_m]
  return (size_t)(hocf::kWsBaseWords + 4 + hocf::kNumQueues + 2 * C * (E + 1) + 3 * (int64_t)E + 2 +
                  cap / tile_m) * 4;
}

static hocf_status a2a_gemm_call(const char* op, bool fused, int P, int E, int e0, int B, int topk, int N, int K,
                                 hocf_dtype in_dt, hocf_dtype out_dt, const void* X, const int32_t* experts,
                                 const void* W, int64_t cap, void* recv, void* Y, int64_t* expert_offsets,
                                 int32_t* dest, int32_t* slot, int64_t* send_counts, int tile_m, int tile_n,
                                 const hocf_sync* sync, void* stream) {
  if (P < 1 || P > HOCF_MAX_P) return fail(HOCF_ERR_INVALID_ARG, "%s: P=%d outside [1, %d]", op, P, HOCF_MAX_P);
  if (E < 1 || E > hocf::kMaxExperts)
    return fail(HOCF_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", op, E, hocf::kMaxExperts);
  if (B < 0 || topk < 0 || N < 0 || K < 0 || cap < 0) return fail(HOCF_ERR_INVALID_ARG, "%s: negative size", op);
  if (!dt_ok(in_dt) || !dt_ok(out_dt)) return fail(HOCF_ERR_INVALID_ARG, "%s: unknown dtype", op);
  if (in_dt != HOCF_BF16) return fail(HOCF_ERR_UNSUPPORTED, "%s: inputs must be bf16", op);
  if ((tile_m != 256 && tile_m != 128) || tile_n != 256)
    return fail(HOCF_ERR_UNSUPPORTED, "%s: tile %dx%d (256x256 or 128x256 only)", op, tile_m, tile_n);
  if (tile_m == 128 && out_dt != HOCF_BF16)
    return fail(HOCF_ERR_UNSUPPORTED, "%s: 128-row tiles take bf16 output only", op);
  if (N % 256 || K % 128)
    return fail(HOCF_ERR_UNSUPPORTED, "%s: N=%d must be a multiple of 256 and K=%d of 128", op, N, K);
  const int oes = out_dt == HOCF_BF16 ? 2 : 4;
  if ((int64_t)P * B * topk >= ((int64_t)1 << 31) || cap >= ((int64_t)1 << 31))
    return fail(HOCF_ERR_UNSUPPORTED, "%s: router entries or receive rows reach 2^31", op);
  if ((int64_t)K * N * 2 >= ((int64_t)1 << 31) || ((int64_t)tile_m * K + K) * 2 >= ((int64_t)1 << 31) ||
      (int64_t)tile_m * N * oes >= ((int64_t)1 << 31))
    return fail(HOCF_ERR_UNSUPPORTED, "%s: an expert's W, a row tile or an output tile reaches 2 GiB", op);
  const size_t need = hocf_a2a_gemm_workspace_bytes(P, E, B, topk, cap, tile_m);
  hocf_status st = check_sync(sync, need);
  if (st != HOCF_OK) return st;
  if (!expert_offsets || !send_counts) return fail(HOCF_ERR_INVALID_ARG, "%s: NULL offsets or send counts", op);
  if ((reinterpret_cast<uintptr_t>(expert_offsets) | reinterpret_cast<uintptr_t>(send_counts)) & 7u)
    return fail(HOCF_ERR_INVALID_ARG, "%s: offsets and send counts must be 8-byte aligned", op);
  if ((int64_t)B * topk > 0) {
    if (!experts) return fail(HOCF_ERR_INVALID_ARG, "%s: NULL router choices", op);
    if (reinterpret_cast<uintptr_t>(experts) & 3u)
      return fail(HOCF_ERR_INVALID_ARG, "%s: router choices must be 4-byte aligned", op);
    if (K > 0 && (!X || !aligned16(X))) return fail(HOCF_ERR_INVALID_ARG, "%s: X NULL or not 16-byte aligned", op);
  }
  if (cap > 0) {
    if (!dest || !slot || ((reinterpret_cast<uintptr_t>(dest) | reinterpret_cast<uintptr_t>(slot)) & 3u))
      return fail(HOCF_ERR_INVALID_ARG, "%s: dest and slot must be 4-byte aligned device arrays", op);
    if (K > 0 && (!recv || !aligned16(recv)))
      return fail(HOCF_ERR_INVALID_ARG, "%s: recv NULL or not 16-byte aligned", op);
    if (N > 0 && (!Y || !aligned16(Y))) return fail(HOCF_ERR_INVALID_ARG, "%s: Y NULL or not 16-byte aligned", op);
    if (N > 0 && K > 0 && (!W || !aligned16(W)))
      return fail(HOCF_ERR_INVALID_ARG, "%s: W NULL or not 16-byte aligned", op);
  }
  {
    Ranges rg;
    rg.in("X", 0, X, (int64_t)P * B * K * 2);
    rg.in("experts", 0, experts, (int64_t)P * B * topk * 4);
    rg.in("W", 0, W, (int64_t)E * K * N * 2);
    rg.out("recv", 0, recv, cap * K * 2);
    rg.out("Y", 0, Y, cap * N * oes);
    rg.out("expert_offsets", 0, expert_offsets, (int64_t)(E + 1) * 8);
    rg.out("dest", 0, dest, cap * 4);
    rg.out("slot", 0, slot, cap * 4);
    rg.out("send_counts", 0, send_counts, (int64_t)P * 8);
    add_sync(rg, sync, need);
    if ((st = rg.check(op)) != HOCF_OK) return st;
  }

  hocf::SyncArgs sa;
  if ((st = to_sync_args(sync, &sa)) != HOCF_OK) return st;
  hocf::A2aGemmArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.experts = experts;
  a.W = static_cast<const uint16_t*>(W);
  a.recv = static_cast<uint16_t*>(recv);
  a.Y = Y;
  a.expert_offsets = expert_offsets;
  a.dest = dest; a.slot = slot;
  a.send_counts = send_counts;
  a.cps = (int)a2g_chunks_per_source(B, topk);
  a.C = P * a.cps;
  uint32_t* w = static_cast<uint32_t*>(sync->workspace) + hocf::kWsBaseWords;
  a.misc = w;
  a.hist = a.misc + 4 + hocf::kNumQueues;
  a.base = a.hist + (int64_t)a.C * (E + 1);
  a.grp = a.base + (int64_t)a.C * (E + 1);
  a.cnt = a.grp + (E + 1);
  a.toff = a.cnt + E;
  a.arrivals = a.toff + (E + 1);
  a.cap = cap;
  a.P = P; a.E = E; a.e0 = e0; a.B = B; a.topk = topk; a.N = N; a.K = K; a.out_dt = out_dt;
  a.tile_m = tile_m;
  a.ntiles = N / tile_n;
  a.nrt = (int)(cap / tile_m);
  a.max_tiles = (int64_t)a.nrt * a.ntiles;
  a.sync = sa;
  return launched(hocf::launch_a2a_gemm(a, fused, static_cast<hipStream_t>(stream)), op);
}

hocf_status hocf_a2a_gemm(int P, int E, int e0, int B, int topk, int N, int K, hocf_dtype in_dt, hocf_dtype out_dt,
                          const void* X, const int32_t* experts, const void* W, int64_t cap, void* recv, void* Y,
                          int64_t* expert_offsets, int32_t* dest, int32_t* slot, int64_t* send_counts, int tile_m,
                          int tile_n, const hocf_sync* sync, void* stream) {
  return a2a_gemm_call("a2a_gemm", true, P, E, e0, B, topk, N, K, in_dt, out_dt, X, experts, W, cap, recv, Y,
                       expert_offsets, dest, slot, send_counts, tile_m, tile_n, sync, stream);
}

hocf_status hocf_a2a_gemm_unfused(int P, int E, int e0, int B, int topk, int N, int K, hocf_dtype in_dt,
                                  hocf_dtype out_dt, const void* X, const int32_t* experts, const void* W,
                                  int64_t cap, void* recv, void* Y, int64_t* expert_offsets, int32_t* dest,
                                  int32_t* slot, int64_t* send_counts, int tile_m, int tile_n, const hocf_sync* sync,
                                  void* stream) {
  return a2a_gemm_call("a2a_gemm_unfused", false, P, E, e0, B, topk, N, K, in_dt, out_dt, X, experts, W, cap, recv,
                       Y, expert_offsets, dest, slot, send_counts, tile_m, tile_n, sync, stream);
}

/* ------------------------------------------------------------ GEMV + AR */

size_t hocf_gemv_ar_workspace_bytes(int P, int N, int tile_n) {
  if (P <= 0 || N < 0 || tile_n <= 0) return 0;
  return (size_t)(hocf::kWsBaseWords + cdiv(N, tile_n)) * 4;
}

// Checks and launch shared by the fused GEMV + AllReduce and its unfused baseline.
static hocf_status gemv_collective(const char* op, bool fused, int P, int Mb, int N, int K, hocf_dtype in_dt,
                                   hocf_dtype slot_dt, hocf_dtype out_dt, const void* x, const void* W,
                                   void* part, uint32_t* part_flags, const hocf_window* win, int tile_n,
                                   const hocf_sync* sync, void* stream) {
  if (P < 1 || P > HOCF_MAX_P) return fail(HOCF_ERR_INVALID_ARG, "%s: P=%d outside [1, %d]", op, P, HOCF_MAX_P);
  if (Mb < 0 || N < 0 || K < 0) return fail(HOCF_ERR_INVALID_ARG, "%s: negative dimension", op);
  if (!dt_ok(in_dt) || !dt_ok(slot_dt) || !dt_ok(out_dt))
    return fail(HOCF_ERR_INVALID_ARG, "%s: unknown dtype", op);
  if (in_dt != HOCF_BF16) return fail(HOCF_ERR_UNSUPPORTED, "%s: inputs must be bf16", op);
  if (Mb > 8) return fail(HOCF_ERR_UNSUPPORTED, "%s: Mb=%d > 8", op, Mb);
  if (tile_n != 128 && tile_n != 256 && tile_n != 512)
    return fail(HOCF_ERR_UNSUPPORTED, "%s: tile_n=%d not in {128, 256, 512}", op, tile_n);
  if (N % 8 || K % 8) return fail(HOCF_ERR_INVALID_ARG, "%s: N and K must be multiples of 8", op);
  // partials and windows are addressed with 32-bit byte offsets
  if ((int64_t)Mb * N * 4 >= ((int64_t)1 << 31))
    return fail(HOCF_ERR_UNSUPPORTED, "%s: Mb * N = %lld elements exceeds 2^29", op, (long long)Mb * N);
  hocf_status st = check_sync(sync, hocf_gemv_ar_workspace_bytes(P, N, tile_n));
  if (st != HOCF_OK) return st;
  if (Mb == 0 || N == 0) return ok();
  if (!x || !W || !part || !part_flags) return fail(HOCF_ERR_INVALID_ARG, "%s: NULL tensor", op);
  if (!aligned16(x) || !aligned16(W) || !aligned16(part))
    return fail(HOCF_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", op);
  if ((st = check_windows(win, P, op)) != HOCF_OK) return st;
  {
    const int ses = slot_dt == HOCF_BF16 ? 2 : 4, oes = out_dt == HOCF_BF16 ? 2 : 4;
    const int64_t nt = cdiv(N, tile_n);
    Ranges rg;
    rg.in("x", 0, x, (int64_t)P * Mb * K * 2);
    rg.in("W", 0, W, (int64_t)P * K * N * 2);
    rg.out("part", 0, part, (int64_t)P * Mb * N * ses);
    rg.out("part_flags", 0, part_flags, (int64_t)P * nt * 4);
    for (int q = 0; q < P; ++q) {
      rg.out("win.data", q, win[q].data, (int64_t)Mb * N * oes);
      rg.out("win.flags", q, win[q].flags, nt * 4);
    }
    add_sync(rg, sync, hocf_gemv_ar_workspace_bytes(P, N, tile_n));
    if ((st = rg.check(op)) != HOCF_OK) return st;
  }

  hocf::SyncArgs sa;
  if ((st = to_sync_args(sync, &sa)) != HOCF_OK) return st;
  hocf::GemvArArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.W = static_cast<const uint16_t*>(W);
  a.part = part; a.part_flags = part_flags;
  for (int q = 0; q < P; ++q) { a.win_data[q] = win[q].data; a.win_flags[q] = win[q].flags; }
  a.ws = static_cast<uint32_t*>(sync->workspace);
  a.P = P; a.Mb = Mb; a.N = N; a.K = K; a.tile_n = tile_n;
  a.ntiles = (int)cdiv(N, tile_n);
  a.slot_dt = slot_dt; a.out_dt = out_dt;
  a.total = (int64_t)P * a.ntiles;
  a.sync = sa;
  a.fused = fused;
  return launched(hocf::launch_gemv_ar(a, static_cast<hipStream_t>(stream)), op);
}

hocf_status hocf_gemv_ar(int P, int Mb, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                         hocf_dtype out_dt, const void* x, const void* W, void* part,
                         uint32_t* part_flags, const hocf_window* win, int tile_n,
                         const hocf_sync* sync, void* stream) {
  return gemv_collective("gemv_ar", true, P, Mb, N, K, in_dt, slot_dt, out_dt, x, W, part, part_flags, win,
                         tile_n, sync, stream);
}

hocf_status hocf_gemv_ar_unfused(int P, int Mb, int N, int K, hocf_dtype in_dt, hocf_dtype slot_dt,
                                 hocf_dtype out_dt, const void* x, const void* W, void* part,
                                 uint32_t* part_flags, const hocf_window* win, int tile_n,
                                 const hocf_sync* sync, void* stream) {
  return gemv_collective("gemv_ar_unfused", false, P, Mb, N, K, in_dt, slot_dt, out_dt, x, W, part, part_flags,
                         win, tile_n, sync, stream);
}

/* ------------------------------------------------------------ AG + GEMM */

size_t hocf_ag_gemm_workspace_bytes(int P) {
  if (P <= 0) return 0;
  return (size_t)(hocf::kWsBaseWords + 2 * (int64_t)P + 3) * 4;
}

hocf_status hocf_ag_gemm(int P, int Mc, int N, int K, hocf_dtype in_dt, hocf_dtype out_dt,
                         const void* A_gathered, const uint32_t* chunk_flags, const void* W,
                         void* out, int tile_m, int tile_n, const hocf_sync* sync, void* stream) {
  if (P < 1 || P > HOCF_MAX_P) return fail(HOCF_ERR_INVALID_ARG, "ag_gemm: P=%d outside [1, %d]", P, HOCF_MAX_P);
  if (Mc < 0 || N < 0 || K < 0) return fail(HOCF_ERR_INVALID_ARG, "ag_gemm: negative dimension");
  if (!dt_ok(in_dt) || !dt_ok(out_dt)) return fail(HOCF_ERR_INVALID_ARG, "ag_gemm: unknown dtype");
  if (in_dt != HOCF_BF16) return fail(HOCF_ERR_UNSUPPORTED, "ag_gemm: inputs must be bf16");
  if (!((tile_m == 256 && tile_n == 256) || (tile_m == 128 && tile_n == 128)))
    return fail(HOCF_ERR_UNSUPPORTED, "ag_gemm: no kernel for tile %dx%d", tile_m, tile_n);
  if (N % 8 || K % 8) return fail(HOCF_ERR_INVALID_ARG, "ag_gemm: N and K must be multiples of 8");
  // output tiles are stored with 32-bit byte offsets from their origin
  if ((int64_t)tile_m * N * (out_dt == HOCF_BF16 ? 2 : 4) >= ((int64_t)1 << 31))
    return fail(HOCF_ERR_UNSUPPORTED, "ag_gemm: tile_m * N * %d bytes per tile row band reach 2 GiB",
                out_dt == HOCF_BF16 ? 2 : 4);
  hocf_status st = check_sync(sync, hocf_ag_gemm_workspace_bytes(P));
  if (st != HOCF_OK) return st;
  if (Mc == 0 || N == 0) return ok();
  if (!A_gathered || !chunk_flags || !W || !out) return fail(HOCF_ERR_INVALID_ARG, "ag_gemm: NULL tensor");
  if ((K && (!aligned16(A_gathered) || !aligned16(W))) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(chunk_flags) & 3u))
    return fail(HOCF_ERR_INVALID_ARG, "ag_gemm: misaligned tensor");
  {
    Ranges rg;
    rg.in("A_gathered", 0, A_gathered, (int64_t)P * Mc * K * 2);
    rg.in("chunk_flags", 0, chunk_flags, (int64_t)P * 4);
    rg.in("W", 0, W, (int64_t)K * N * 2);
    rg.out("out", 0, out, (int64_t)P * Mc * N * (out_dt == HOCF_BF16 ? 2 : 4));
    add_sync(rg, sync, hocf_ag_gemm_workspace_bytes(P));
    if ((st = rg.check("ag_gemm")) != HOCF_OK) return st;
  }

  hocf::SyncArgs sa;
  if ((st = to_sync_args(sync, &sa)) != HOCF_OK) return st;
  hocf::AgGemmArgs a{};
  a.A = static_cast<const uint16_t*>(A_gathered);
  a.chunk_flags = chunk_flags;
  a.W = static_cast<const uint16_t*>(W);
  a.out = out;
  a.ws = static_cast<uint32_t*>(sync->workspace);
  a.P = P; a.Mc = Mc; a.N = N; a.K = K; a.out_dt = out_dt;
  a.mtiles = (int)cdiv(Mc, tile_m);
  a.ntiles = (int)cdiv(N, tile_n);
  a.sync = sa;
  return launched(hocf::launch_ag_gemm(a, tile_m, tile_n, static_cast<hipStream_t>(stream)), "ag_gemm");
}

/* ------------------------------------------------------------ emb-bag + A2A */

size_t hocf_embbag_a2a_workspace_bytes(void) { return (size_t)hocf::kWsBaseWords * 4; }

hocf_status hocf_embbag_a2a(int T, int64_t R, int D, int B, int L, int P, const float* tables,
                            const int32_t* indices, const int64_t* offsets,
                            const hocf_window* win, int tile_bags, const hocf_sync* sync,
                            void* stream) {
  if (P < 1 || P > HOCF_MAX_P) return fail(HOCF_ERR_INVALID_ARG, "embbag_a2a: P=%d outside [1, %d]", P, HOCF_MAX_P);
  if (T < 0 || R < 0 || D < 0 || B < 0 || (!offsets && L < 0))
    return fail(HOCF_ERR_INVALID_ARG, "embbag_a2a: negative dimension");
  if (B % P) return fail(HOCF_ERR_INVALID_ARG, "embbag_a2a: B=%d not divisible by P=%d", B, P);
  if (D % 4) return fail(HOCF_ERR_INVALID_ARG, "embbag_a2a: D=%d not a multiple of 4", D);
  if (D > 512) return fail(HOCF_ERR_UNSUPPORTED, "embbag_a2a: D=%d > 512", D);
  if (tile_bags < 1 || tile_bags > 4096)
    return fail(HOCF_ERR_INVALID_ARG, "embbag_a2a: tile_bags=%d outside [1, 4096]", tile_bags);
  if ((int64_t)tile_bags * T * D * 4 >= (int64_t(1) << 31))
    return fail(HOCF_ERR_UNSUPPORTED, "embbag_a2a: a tile's window rows (tile_bags*T*D*4 bytes) reach 2 GiB");
  hocf_status st = check_sync(sync, hocf_embbag_a2a_workspace_bytes());
  if (st != HOCF_OK) return st;
  if (T == 0 || B == 0 || D == 0) return ok();
  if (!tables && R > 0) return fail(HOCF_ERR_INVALID_ARG, "embbag_a2a: NULL tables");
  if (!indices && (offsets || L > 0)) return fail(HOCF_ERR_INVALID_ARG, "embbag_a2a: NULL indices");
  if ((tables && !aligned16(tables)) || (offsets && (reinterpret_cast<uintptr_t>(offsets) & 7u)))
    return fail(HOCF_ERR_INVALID_ARG, "embbag_a2a: misaligned tensor");
  if ((st = check_windows(win, P, "embbag_a2a")) != HOCF_OK) return st;
  {
    const int64_t Bd = B / P, nj = cdiv(Bd, tile_bags);
    Ranges rg;
    rg.in("tables", 0, tables, (int64_t)T * R * D * 4);
    // (with CSR offsets the extent of `indices` is only known on the device)
    if (!offsets) rg.in("indices", 0, indices, (int64_t)T * B * L * 4);
    rg.in("offsets", 0, offsets, offsets ? ((int64_t)T * B + 1) * 8 : 0);
    for (int d = 0; d < P; ++d) {
      rg.out("win.data", d, win[d].data, Bd * T * D * 4);
      rg.out("win.flags", d, win[d].flags, (int64_t)T * nj * 4);
    }
    add_sync(rg, sync, hocf_embbag_a2a_workspace_bytes());
    if ((st = rg.check("embbag_a2a")) != HOCF_OK) return st;
  }

  hocf::SyncArgs sa;
  if ((st = to_sync_args(sync, &sa)) != HOCF_OK) return st;
  hocf::EmbbagArgs a{};
  a.tables = tables; a.indices = indices; a.offsets = offsets;
  for (int d = 0; d < P; ++d) {
    a.win_data[d] = static_cast<float*>(win[d].data);
    a.win_flags[d] = win[d].flags;
  }
  a.ws = static_cast<uint32_t*>(sync->workspace);
  a.R = R; a.T = T; a.D = D; a.B = B; a.L = offsets ? 0 : L; a.P = P;
  a.Bd = B / P; a.tile_bags = tile_bags;
  a.nj = (int)cdiv(a.Bd, tile_bags);
  a.total = (int64_t)T * P * a.nj;
  a.sync = sa;
  return launched(hocf::launch_embbag_a2a(a, static_cast<hipStream_t>(stream)), "embbag_a2a");
}

/* ------------------------------------------------------------ copy-engine puts */

// One device pointer of the current device, checked with the runtime.
static hocf_status device_range(const char* what, int idx, const void* p, int dev) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // the query's error is ours to clear
    return fail(HOCF_ERR_INVALID_ARG, "dma_put: %s[%d] is not memory the HIP runtime knows", what, idx);
  }
  if (at.type != hipMemoryTypeDevice || at.device != dev)
    return fail(HOCF_ERR_INVALID_ARG, "dma_put: %s[%d] is not device memory of device %d", what, idx, dev);
  return HOCF_OK;
}

hocf_status hocf_dma_put(int n, const void* const* src, void* const* dst, const int64_t* bytes,
                         uint32_t* const* signal, const uint32_t* signal_value, hocf_engine engine,
                         void* stream) {
  if (n < 0 || n > HOCF_MAX_PUTS) return fail(HOCF_ERR_INVALID_ARG, "dma_put: n=%d outside [0, %d]", n, HOCF_MAX_PUTS);
  if (engine != HOCF_ENGINE_DMA && engine != HOCF_ENGINE_CU)
    return fail(HOCF_ERR_INVALID_ARG, "dma_put: unknown engine %d", (int)engine);
  if (n == 0) return ok();
  if (!src || !dst || !bytes) return fail(HOCF_ERR_INVALID_ARG, "dma_put: NULL argument array");
  bool signals = false;
  for (int i = 0; signal && i < n; ++i) signals = signals || signal[i];
  if (signals && (!signal_value || (reinterpret_cast<uintptr_t>(signal_value) & 3u)))
    return fail(HOCF_ERR_INVALID_ARG, "dma_put: signal_value NULL or not 4-byte aligned");
  hocf_status st;
  {
    Ranges rg;
    if (signals) rg.in("signal_value", 0, signal_value, 4);
    for (int i = 0; i < n; ++i) {
      if (bytes[i] < 0) return fail(HOCF_ERR_INVALID_ARG, "dma_put: bytes[%d] < 0", i);
      if (bytes[i] > 0 && (!src[i] || !dst[i])) return fail(HOCF_ERR_INVALID_ARG, "dma_put: put %d has a NULL buffer", i);
      if (bytes[i] > 0 && (!aligned16(src[i]) || !aligned16(dst[i])))
        return fail(HOCF_ERR_INVALID_ARG, "dma_put: put %d misaligned (16 bytes)", i);
      if (signal && signal[i] && (reinterpret_cast<uintptr_t>(signal[i]) & 3u))
        return fail(HOCF_ERR_INVALID_ARG, "dma_put: signal[%d] not 4-byte aligned", i);
      rg.in("src", i, src[i], bytes[i]);
      rg.out("dst", i, dst[i], bytes[i]);
      if (signal) rg.out("signal", i, signal[i], 4);
    }
    if ((st = rg.check("dma_put")) != HOCF_OK) return st;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(HOCF_ERR_HIP, "dma_put: no current HIP device");
  if (signals && (st = device_range("signal_value", 0, signal_value, dev)) != HOCF_OK) return st;
  for (int i = 0; i < n; ++i) {
    if (bytes[i] > 0 && ((st = device_range("src", i, src[i], dev)) != HOCF_OK ||
                         (st = device_range("dst", i, dst[i], dev)) != HOCF_OK))
      return st;
    if (signal && signal[i] && (st = device_range("signal", i, signal[i], dev)) != HOCF_OK) return st;
  }

  // Each put is one or two copies on the stream: the bytes, then the signal
  // word.  The stream orders them (each starts once the one before it has
  // completed), so a consumer that sees the signal sees the bytes.  Asked for
  // the DMA engine, the runtime moves a copy of 64 KB or more on a copy
  // (SDMA) engine; it runs smaller ones, and so every signal, as its own
  // one-workgroup copy kernel.  Asked for the CU engine, it runs its copy
  // kernels throughout.
  const hipMemcpyKind kind = engine == HOCF_ENGINE_DMA ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipSuccess;
    if (bytes[i] > 0) e = hipMemcpyAsync(dst[i], src[i], (size_t)bytes[i], kind, s);
    if (e == hipSuccess && signal && signal[i]) e = hipMemcpyAsync(signal[i], signal_value, 4, kind, s);
    if (e != hipSuccess) return fail(HOCF_ERR_HIP, "dma_put: put %d of %d: %s (puts before it stay enqueued)", i, n, hipGetErrorString(e));
  }
  return ok();
}

}  // extern "C"
