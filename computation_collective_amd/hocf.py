"""Python binding of libhocf.so (argument marshalling only).

The functions below carry the names and arguments of the C entry points in
``include/hocf.h``; every step of the computation runs in the library's HIP
kernels.  Tensor arguments may be ``torch`` tensors (their device pointer is
passed) or raw integer addresses.  PyTorch is used only to own device memory
and streams.  Importing this module does not touch the GPU; the first call
loads the library and fails loudly if it has not been built.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhocf.so")
TRACE_LIB_PATH = os.path.join(HERE, "libhocf_trace.so")

HOCF_OK = 0
HOCF_ERR_INVALID_ARG = 1
HOCF_ERR_UNSUPPORTED = 2
HOCF_ERR_HIP = 3
HOCF_ERR_TIMEOUT = 4
HOCF_ERR_ABORTED = 5
HOCF_ERR_BAD_INDEX = 6
HOCF_ERR_PROTOCOL = 7
HOCF_ERR_CAPACITY = 8
HOCF_F32 = 0
HOCF_BF16 = 1
HOCF_MAX_P = 16

EXPORTED = [
    "hocf_gemm_rs", "hocf_gemm_rs_workspace_bytes", "hocf_gemm_rs_noalloc", "hocf_gemm_rs_decomposed",
    "hocf_gemm_ar", "hocf_gemm_ar_workspace_bytes", "hocf_gemm_rs_unfused",
    "hocf_gemv_ar", "hocf_gemv_ar_workspace_bytes", "hocf_gemv_ar_unfused",
    "hocf_ag_gemm", "hocf_ag_gemm_workspace_bytes",
    "hocf_embbag_a2a", "hocf_embbag_a2a_workspace_bytes",
    "hocf_gemm_a2a", "hocf_gemm_a2a_workspace_bytes",
    "hocf_a2a_gemm", "hocf_a2a_gemm_unfused", "hocf_a2a_gemm_workspace_bytes",
    "hocf_dma_put",
    "hocf_status_string", "hocf_last_error", "hocf_abi_version",
]


class hocf_window(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("flags", ctypes.c_void_p)]


class hocf_sync(ctypes.Structure):
    _fields_ = [("epoch", ctypes.c_uint32), ("status", ctypes.c_void_p),
                ("abort_flag", ctypes.c_void_p), ("spin_timeout_ns", ctypes.c_uint64),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class HocfError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)} ({status}): {detail}")
        self.status = status


_lib = None


def use_trace_library() -> None:
    """Load the trace build (libhocf_trace.so: the GEMM + ReduceScatter /
    AllReduce kernel records per-iteration timestamps into its workspace, and
    their workspace queries ask for room for them) instead of the product
    library.  Must be called before the first call into the library."""
    global LIB_PATH
    if _lib is not None and LIB_PATH != TRACE_LIB_PATH:
        raise RuntimeError("the product library is already loaded")
    LIB_PATH = TRACE_LIB_PATH


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with computation_collective_amd/build.py "
                               "(the fused operators have no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        i, i64, vp, sz, u32 = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32
        W = ctypes.POINTER(hocf_window)
        S = ctypes.POINTER(hocf_sync)
        L.hocf_gemm_rs.argtypes = [i, i, i, i, i, i, i, vp, vp, W, vp, i, i, S, vp]
        L.hocf_gemm_rs_workspace_bytes.argtypes = [i, i, i, i, i]
        L.hocf_gemm_rs_unfused.argtypes = [i, i, i, i, i, i, i, vp, vp, W, vp, i, i, S, vp]
        L.hocf_gemm_rs_noalloc.argtypes = [i, i, i, i, i, i, i, vp, vp, W, vp, i, i, S, vp]
        L.hocf_gemm_rs_decomposed.argtypes = [i, i, i, i, i, i, i, vp, vp, W, vp, i, i, i, i, S, vp, vp]
        L.hocf_gemm_rs_decomposed.restype = i
        L.hocf_gemm_ar.argtypes = [i, i, i, i, i, i, i, vp, vp, W, ctypes.POINTER(vp), i, i, S, vp]
        L.hocf_gemm_ar_workspace_bytes.argtypes = [i, i, i, i, i]
        L.hocf_gemv_ar.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, vp, W, i, S, vp]
        L.hocf_gemv_ar_workspace_bytes.argtypes = [i, i, i]
        L.hocf_gemv_ar_unfused.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, vp, W, i, S, vp]
        L.hocf_ag_gemm.argtypes = [i, i, i, i, i, i, vp, vp, vp, vp, i, i, S, vp]
        L.hocf_ag_gemm_workspace_bytes.argtypes = [i]
        L.hocf_embbag_a2a.argtypes = [i, i64, i, i, i, i, vp, vp, vp, W, i, S, vp]
        L.hocf_embbag_a2a_workspace_bytes.argtypes = []
        L.hocf_gemm_a2a.argtypes = [i, i, i64, i, i, i, i, vp, vp, vp, vp, vp, vp, W, i64, i, i, S, vp]
        L.hocf_gemm_a2a_workspace_bytes.argtypes = [i]
        for f in ("hocf_a2a_gemm", "hocf_a2a_gemm_unfused"):
            getattr(L, f).argtypes = [i] * 9 + [vp] * 3 + [i64] + [vp] * 6 + [i, i, S, vp]
            getattr(L, f).restype = i
        L.hocf_a2a_gemm_workspace_bytes.argtypes = [i, i, i, i, i64, i]
        L.hocf_a2a_gemm_workspace_bytes.restype = sz
        for f in ("hocf_gemm_rs", "hocf_gemm_rs_unfused", "hocf_gemm_rs_noalloc", "hocf_gemm_ar", "hocf_gemv_ar", "hocf_gemv_ar_unfused", "hocf_ag_gemm",
                  "hocf_embbag_a2a", "hocf_gemm_a2a"):
            getattr(L, f).restype = i
        for f in ("hocf_gemm_rs_workspace_bytes", "hocf_gemm_ar_workspace_bytes", "hocf_gemv_ar_workspace_bytes",
                  "hocf_ag_gemm_workspace_bytes", "hocf_embbag_a2a_workspace_bytes",
                  "hocf_gemm_a2a_workspace_bytes"):
            getattr(L, f).restype = sz
        PV = ctypes.POINTER(vp)
        L.hocf_dma_put.argtypes = [i, PV, PV, ctypes.POINTER(i64), PV, vp, i, vp]
        L.hocf_dma_put.restype = i
        L.hocf_status_string.argtypes = [i]
        L.hocf_status_string.restype = ctypes.c_char_p
        L.hocf_last_error.argtypes = []
        L.hocf_last_error.restype = ctypes.c_char_p
        L.hocf_abi_version.restype = i
        _lib = L
    return _lib


def ptr(x) -> int | None:
    """Device address of a torch tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def windows(pairs) -> ctypes.Array:
    """Host array of hocf_window from [(data, flags), ...]."""
    arr = (hocf_window * len(pairs))()
    for k, (d, f) in enumerate(pairs):
        arr[k].data = ptr(d)
        arr[k].flags = ptr(f)
    return arr


def pointers(xs) -> ctypes.Array | None:
    """Host array of device pointers from [tensor or int, ...] (None passes through)."""
    if xs is None:
        return None
    return (ctypes.c_void_p * len(xs))(*[ptr(x) for x in xs])


def sync(epoch, workspace, workspace_bytes, status=None, abort_flag=None, spin_timeout_ns=0):
    s = hocf_sync()
    s.epoch = epoch
    s.status = ptr(status)
    s.abort_flag = ptr(abort_flag)
    s.spin_timeout_ns = spin_timeout_ns
    s.workspace = ptr(workspace)
    s.workspace_bytes = workspace_bytes
    return s


def status_string(st: int) -> str:
    return lib().hocf_status_string(st).decode()


def last_error() -> str:
    return lib().hocf_last_error().decode()


def check(st: int) -> None:
    if st != HOCF_OK:
        raise HocfError(st, last_error())


def hocf_abi_version() -> int:
    return lib().hocf_abi_version()


def hocf_gemm_rs_workspace_bytes(P, M, N, tile_m, tile_n) -> int:
    return lib().hocf_gemm_rs_workspace_bytes(P, M, N, tile_m, tile_n)


def hocf_gemm_ar_workspace_bytes(P, M, N, tile_m, tile_n) -> int:
    return lib().hocf_gemm_ar_workspace_bytes(P, M, N, tile_m, tile_n)


def hocf_gemv_ar_workspace_bytes(P, N, tile_n) -> int:
    return lib().hocf_gemv_ar_workspace_bytes(P, N, tile_n)


def hocf_ag_gemm_workspace_bytes(P) -> int:
    return lib().hocf_ag_gemm_workspace_bytes(P)


def hocf_embbag_a2a_workspace_bytes() -> int:
    return lib().hocf_embbag_a2a_workspace_bytes()


def hocf_gemm_rs(P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, out, tile_m, tile_n, sync_,
                 stream=None) -> int:
    return lib().hocf_gemm_rs(P, M, N, K, in_dt, slot_dt, out_dt, ptr(A), ptr(W), win, ptr(out),
                              tile_m, tile_n, ctypes.byref(sync_), _stream(stream))


def hocf_gemm_rs_unfused(P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, out, tile_m, tile_n, sync_,
                         stream=None) -> int:
    return lib().hocf_gemm_rs_unfused(P, M, N, K, in_dt, slot_dt, out_dt, ptr(A), ptr(W), win, ptr(out),
                                      tile_m, tile_n, ctypes.byref(sync_), _stream(stream))


def hocf_gemm_rs_noalloc(P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, out, tile_m, tile_n, sync_,
                         stream=None) -> int:
    """sync_.workspace must be None (the library's own scratch is used)."""
    return lib().hocf_gemm_rs_noalloc(P, M, N, K, in_dt, slot_dt, out_dt, ptr(A), ptr(W), win, ptr(out),
                                      tile_m, tile_n, ctypes.byref(sync_), _stream(stream))


HOCF_NOALLOC_SCRATCH_BYTES = 1 << 20


def hocf_gemm_rs_decomposed(P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, out, tile_m, tile_n, pieces, fold_cus,
                            sync_, stream=None, coll_stream=None) -> int:
    return lib().hocf_gemm_rs_decomposed(P, M, N, K, in_dt, slot_dt, out_dt, ptr(A), ptr(W), win, ptr(out),
                                         tile_m, tile_n, pieces, fold_cus, ctypes.byref(sync_), _stream(stream),
                                         _stream(coll_stream))


def hocf_gemm_ar(P, M, N, K, in_dt, slot_dt, out_dt, A, W, win, outs, tile_m, tile_n, sync_,
                 stream=None) -> int:
    """outs: P device buffers (or a host pointer array from pointers())."""
    arr = outs if outs is None or isinstance(outs, ctypes.Array) else pointers(outs)
    return lib().hocf_gemm_ar(P, M, N, K, in_dt, slot_dt, out_dt, ptr(A), ptr(W), win, arr,
                              tile_m, tile_n, ctypes.byref(sync_), _stream(stream))


def hocf_gemv_ar(P, Mb, N, K, in_dt, slot_dt, out_dt, x, W, part, part_flags, win, tile_n, sync_,
                 stream=None) -> int:
    return lib().hocf_gemv_ar(P, Mb, N, K, in_dt, slot_dt, out_dt, ptr(x), ptr(W), ptr(part),
                              ptr(part_flags), win, tile_n, ctypes.byref(sync_), _stream(stream))


def hocf_gemv_ar_unfused(P, Mb, N, K, in_dt, slot_dt, out_dt, x, W, part, part_flags, win, tile_n, sync_,
                         stream=None) -> int:
    return lib().hocf_gemv_ar_unfused(P, Mb, N, K, in_dt, slot_dt, out_dt, ptr(x), ptr(W), ptr(part),
                                      ptr(part_flags), win, tile_n, ctypes.byref(sync_), _stream(stream))


def hocf_ag_gemm(P, Mc, N, K, in_dt, out_dt, A_gathered, chunk_flags, W, out, tile_m, tile_n,
                 sync_, stream=None) -> int:
    return lib().hocf_ag_gemm(P, Mc, N, K, in_dt, out_dt, ptr(A_gathered), ptr(chunk_flags),
                              ptr(W), ptr(out), tile_m, tile_n, ctypes.byref(sync_), _stream(stream))


HOCF_ENGINE_DMA, HOCF_ENGINE_CU = 0, 1
HOCF_MAX_PUTS = 16


def hocf_dma_put(src, dst, nbytes, signal, signal_value, engine, stream=None) -> int:
    """Puts i = 0..n-1 on `stream`: nbytes[i] bytes src[i] -> dst[i], then the word
    at signal_value -> signal[i] (tensors or device addresses; src/dst may be None
    where nbytes[i] == 0)."""
    n = len(nbytes)
    return lib().hocf_dma_put(n, pointers(src), pointers(dst), (ctypes.c_int64 * n)(*[int(b) for b in nbytes]),
                              pointers(signal), ptr(signal_value), engine, _stream(stream))


def hocf_embbag_a2a(T, R, D, B, L, P, tables, indices, offsets, win, tile_bags, sync_,
                    stream=None) -> int:
    return lib().hocf_embbag_a2a(T, R, D, B, L, P, ptr(tables), ptr(indices), ptr(offsets), win,
                                 tile_bags, ctypes.byref(sync_), _stream(stream))


def hocf_gemm_a2a_workspace_bytes(P) -> int:
    return lib().hocf_gemm_a2a_workspace_bytes(P)


def hocf_a2a_gemm_workspace_bytes(P, E, B, topk, cap, tile_m) -> int:
    return lib().hocf_a2a_gemm_workspace_bytes(P, E, B, topk, cap, tile_m)


def hocf_a2a_gemm(P, E, e0, B, topk, N, K, in_dt, out_dt, X, experts, W, cap, recv, Y, expert_offsets, dest,
                  slot, send_counts, tile_m, tile_n, sync_, stream=None, unfused=False) -> int:
    """All-to-All + GEMM (MoE dispatch + GEMM); every array a device buffer."""
    fn = lib().hocf_a2a_gemm_unfused if unfused else lib().hocf_a2a_gemm
    return fn(P, E, e0, B, topk, N, K, in_dt, out_dt, ptr(X), ptr(experts), ptr(W), cap, ptr(recv), ptr(Y),
              ptr(expert_offsets), ptr(dest), ptr(slot), ptr(send_counts), tile_m, tile_n, ctypes.byref(sync_),
              _stream(stream))


def _host_i64(a):
    """A host int64 array for the call (kept alive by the caller's reference)."""
    import numpy as np
    if a is None:
        return None
    arr = np.ascontiguousarray(a, dtype=np.int64)
    return arr


def hocf_gemm_a2a(P, E, T, N, K, in_dt, out_dt, X, W, expert_offsets, dest, slot, send_counts, win, cap,
                  tile_m, tile_n, sync_, stream=None) -> int:
    """expert_offsets, send_counts: host int64 sequences; the rest device buffers."""
    off = _host_i64(expert_offsets)
    cnt = _host_i64(send_counts)
    return lib().hocf_gemm_a2a(P, E, T, N, K, in_dt, out_dt, ptr(X), ptr(W),
                               None if off is None else off.ctypes.data, ptr(dest), ptr(slot),
                               None if cnt is None else cnt.ctypes.data, win, cap, tile_m, tile_n,
                               ctypes.byref(sync_), _stream(stream))


# --------------------------------------------------------------- chunk releasers
# The AllGather side of hocf_ag_gemm.  On ROCm a stream write-value is a tiny
# blit kernel, ordered with the rest of its stream; a release stream that
# shares a hardware queue with the consumer's stream would queue behind the
# consumer kernel that waits for it.  So flags are either written on the
# consumer's own stream before the kernel, or by the host into coherent
# pinned memory while the kernel runs.

_hip = None


def _hip_runtime():
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (loads the HIP runtime torch was built with)
        for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise RuntimeError("HIP runtime library not found")
        _hip.hipStreamWriteValue32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32,
                                               ctypes.c_uint]
        _hip.hipStreamWriteValue32.restype = ctypes.c_int
        _hip.hipStreamWaitValue32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32,
                                              ctypes.c_uint, ctypes.c_uint32]
        _hip.hipStreamWaitValue32.restype = ctypes.c_int
        _hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        _hip.hipHostMalloc.restype = ctypes.c_int
    return _hip


HIP_STREAM_WAIT_VALUE_GTE = 0x0
HIP_HOST_MALLOC_MAPPED = 0x2
HIP_HOST_MALLOC_COHERENT = 0x40000000
_host_blocks = []   # coherent host blocks live until the process ends


def host_coherent(nbytes: int):
    """Pinned, device-mapped, coherent host memory (fine-grained: the GPU does not
    cache it), e.g. for flags or chunks written by the host while a kernel runs.
    Returns (address, ctypes buffer).  Kept until the process ends."""
    import ctypes as C
    hip = _hip_runtime()
    p = C.c_void_p()
    rc = hip.hipHostMalloc(C.byref(p), C.c_size_t(nbytes), HIP_HOST_MALLOC_COHERENT | HIP_HOST_MALLOC_MAPPED)
    if rc != 0:
        raise RuntimeError(f"hipHostMalloc failed ({rc})")
    buf = (C.c_char * nbytes).from_address(p.value)
    C.memset(p.value, 0, nbytes)
    _host_blocks.append((p, buf))
    return p.value, buf


def stream_write_value32(stream, address: int, value: int) -> None:
    """Enqueue a 32-bit write of `value` at device address `address` on `stream`."""
    rc = _hip_runtime().hipStreamWriteValue32(_stream(stream), address, value, 0)
    if rc != 0:
        raise RuntimeError(f"hipStreamWriteValue32 failed ({rc})")


def stream_wait_value32(stream, address: int, value: int) -> None:
    """Enqueue a wait on `stream` until the word at `address` is >= `value`."""
    rc = _hip_runtime().hipStreamWaitValue32(_stream(stream), address, value,
                                             HIP_STREAM_WAIT_VALUE_GTE, 0xFFFFFFFF)
    if rc != 0:
        raise RuntimeError(f"hipStreamWaitValue32 failed ({rc})")


def release_chunks(stream, chunk_flags, order, epoch) -> None:
    """Set chunk_flags[c] = epoch for c in `order`, each after the previous, on `stream`."""
    base = ptr(chunk_flags)
    for c in order:
        stream_write_value32(stream, base + 4 * int(c), epoch)

