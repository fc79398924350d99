"""CPU oracle for the fused computation + collective-epilogue operators.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``, never by the product path.  It
shares no code with the HIP library; it is a thin ctypes wrapper over
``oracle.c`` (plain C, fp64 accumulation, fixed rank-order fp32 folds).

Data types: 0 = fp32 (numpy float32), 1 = bf16 carried as numpy uint16 bit
patterns.  Every array argument must be C-contiguous.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.oracle_gemm_rs.argtypes = [i32] * 7 + [vp] * 4
        lib.oracle_gemm_rs_points.argtypes = [i32] * 7 + [vp, vp, i64, vp, vp, vp, vp]
        lib.oracle_gemv_ar.argtypes = [i32] * 7 + [vp] * 4
        lib.oracle_gemm_ar.argtypes = [i32] * 7 + [vp] * 4
        lib.oracle_gemm_a2a.argtypes = [i32, i32, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, i64, vp]
        lib.oracle_ag_gemm.argtypes = [i32] * 6 + [vp] * 4
        lib.oracle_a2a_gemm.argtypes = [i32] * 9 + [vp] * 3 + [i32, i64] + [vp] * 6
        lib.oracle_a2a_gemm.restype = ctypes.c_int
        lib.oracle_ag_gemm_points.argtypes = [i32] * 6 + [vp, vp, i64, vp, vp, vp]
        lib.oracle_embbag_a2a.argtypes = [i32, i64, i32, i32, i32, i32, vp, vp, vp, vp]
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_max_threads.restype = i32
        for f in (lib.oracle_gemm_rs, lib.oracle_gemm_rs_points, lib.oracle_gemv_ar,
                  lib.oracle_ag_gemm, lib.oracle_ag_gemm_points, lib.oracle_embbag_a2a):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _np_dt(dt):
    return np.uint16 if dt == BF16 else np.float32


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(dt, *arrays):
    for a in arrays:
        assert a.dtype == _np_dt(dt), f"expected {_np_dt(dt)}, got {a.dtype}"


def set_threads(n: int) -> None:
    """Number of OpenMP threads the oracle uses from now on."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    """Threads the oracle's parallel regions will use."""
    return int(_load().oracle_max_threads())


def gemm_rs(P, M, N, K, in_dt, slot_dt, out_dt, A, W, want_slots=True):
    """GEMM + ReduceScatter.  Returns (slots [P][P][Mc][N] or None, out [M][N])."""
    _check(in_dt, A, W)
    assert A.shape == (P, M, K) and W.shape == (P, K, N)
    Mc = M // P
    slots = np.empty((P, P, Mc, N), dtype=_np_dt(slot_dt)) if want_slots else None
    out = np.empty((M, N), dtype=_np_dt(out_dt))
    rc = _load().oracle_gemm_rs(P, M, N, K, in_dt, slot_dt, out_dt, _ptr(A), _ptr(W),
                                _ptr(slots), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_gemm_rs rejected its arguments (rc={rc})")
    return slots, out


def gemm_rs_points(P, M, N, K, in_dt, slot_dt, out_dt, A, W, ms, ns):
    """Sampled GEMM + ReduceScatter at (ms[i], ns[i]).  Returns (slot_vals [n][P], out_vals [n])."""
    _check(in_dt, A, W)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    sv = np.empty((len(ms), P), dtype=_np_dt(slot_dt))
    ov = np.empty(len(ms), dtype=_np_dt(out_dt))
    rc = _load().oracle_gemm_rs_points(P, M, N, K, in_dt, slot_dt, out_dt, _ptr(A), _ptr(W),
                                       len(ms), _ptr(ms), _ptr(ns), _ptr(sv), _ptr(ov))
    if rc != 0:
        raise ValueError(f"oracle_gemm_rs_points rejected its arguments (rc={rc})")
    return sv, ov


def gemm_ar(P, M, N, K, in_dt, slot_dt, out_dt, A, W, want_slots=True):
    """GEMM + AllReduce.  Returns (slots [P][P][Mc][N] or None, win [P][M][N])."""
    _check(in_dt, A, W)
    assert A.shape == (P, M, K) and W.shape == (P, K, N)
    Mc = M // P
    slots = np.empty((P, P, Mc, N), dtype=_np_dt(slot_dt)) if want_slots else None
    win = np.empty((P, M, N), dtype=_np_dt(out_dt))
    rc = _load().oracle_gemm_ar(P, M, N, K, in_dt, slot_dt, out_dt, _ptr(A), _ptr(W),
                                _ptr(slots), _ptr(win))
    if rc != 0:
        raise ValueError(f"oracle_gemm_ar rejected its arguments (rc={rc})")
    return slots, win


def gemm_a2a(P, E, N, K, in_dt, out_dt, X, W, offsets, dest, slot, cap, win=None):
    """GEMM + All-to-All.  Returns win [P][cap][N]: row i of the expert GEMM at
    [dest[i]][slot[i]]; entries no row names keep their previous contents
    (`win`, or zeros)."""
    _check(in_dt, X, W)
    T = X.shape[0]
    assert X.shape == (T, K) and W.shape == (E, K, N)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    dest = np.ascontiguousarray(dest, dtype=np.int32)
    slot = np.ascontiguousarray(slot, dtype=np.int32)
    assert offsets.shape == (E + 1,) and dest.shape == (T,) and slot.shape == (T,)
    if win is None:
        win = np.zeros((P, cap, N), dtype=_np_dt(out_dt))
    rc = _load().oracle_gemm_a2a(P, E, T, N, K, in_dt, out_dt, _ptr(X), _ptr(W), _ptr(offsets), _ptr(dest),
                                 _ptr(slot), cap, _ptr(win))
    if rc != 0:
        raise ValueError(f"oracle_gemm_a2a rejected its arguments (rc={rc})")
    return win


def a2a_gemm(P, E, e0, B, topk, N, K, in_dt, out_dt, X, experts, W, tile_m, cap, recv=None, Y=None,
             dest=None, slot=None):
    """All-to-All + GEMM (MoE dispatch + GEMM), this rank owning experts e0 .. e0+E-1.
    Returns (recv [cap][K], Y [cap][N], offsets [E+1], dest [cap], slot [cap], send_counts [P]);
    rows from offsets[E] on keep the contents of the arrays passed in (or zeros / -1)."""
    _check(in_dt, X, W)
    assert X.shape == (P, B, K) and W.shape == (E, K, N)
    experts = np.ascontiguousarray(experts, dtype=np.int32)
    assert experts.shape == (P, B, topk)
    if recv is None:
        recv = np.zeros((cap, K), dtype=_np_dt(in_dt))
    if Y is None:
        Y = np.zeros((cap, N), dtype=_np_dt(out_dt))
    if dest is None:
        dest = np.full(cap, -1, dtype=np.int32)
    if slot is None:
        slot = np.full(cap, -1, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int64)
    send_counts = np.zeros(P, dtype=np.int64)
    rc = _load().oracle_a2a_gemm(P, E, e0, B, topk, N, K, in_dt, out_dt, _ptr(X), _ptr(experts), _ptr(W),
                                 tile_m, cap, _ptr(recv), _ptr(Y), _ptr(offsets), _ptr(dest), _ptr(slot),
                                 _ptr(send_counts))
    if rc != 0:
        raise ValueError(f"oracle_a2a_gemm rejected its arguments (rc={rc})")
    return recv, Y, offsets, dest, slot, send_counts


def gemv_ar(P, Mb, N, K, in_dt, slot_dt, out_dt, x, W):
    """GEMV + AllReduce.  Returns (part [P][Mb][N], win [P][Mb][N])."""
    _check(in_dt, x, W)
    assert x.shape == (P, Mb, K) and W.shape == (P, K, N)
    part = np.empty((P, Mb, N), dtype=_np_dt(slot_dt))
    win = np.empty((P, Mb, N), dtype=_np_dt(out_dt))
    rc = _load().oracle_gemv_ar(P, Mb, N, K, in_dt, slot_dt, out_dt, _ptr(x), _ptr(W),
                                _ptr(part), _ptr(win))
    if rc != 0:
        raise ValueError(f"oracle_gemv_ar rejected its arguments (rc={rc})")
    return part, win


def _chunk_ptrs(chunks):
    return (ctypes.c_void_p * len(chunks))(*[_ptr(c) for c in chunks])


def ag_gemm(P, Mc, N, K, in_dt, out_dt, chunks, W):
    """AllGather + GEMM.  chunks: list of P arrays [Mc][K] (rank c's chunk).
    Returns (gathered [P*Mc][K], out [P*Mc][N])."""
    assert len(chunks) == P
    _check(in_dt, W, *chunks)
    g = np.empty((P * Mc, K), dtype=_np_dt(in_dt))
    out = np.empty((P * Mc, N), dtype=_np_dt(out_dt))
    cp = _chunk_ptrs(chunks)
    rc = _load().oracle_ag_gemm(P, Mc, N, K, in_dt, out_dt, cp, _ptr(W), _ptr(g), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_ag_gemm rejected its arguments (rc={rc})")
    return g, out


def ag_gemm_points(P, Mc, N, K, in_dt, out_dt, chunks, W, ms, ns):
    assert len(chunks) == P
    _check(in_dt, W, *chunks)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    ov = np.empty(len(ms), dtype=_np_dt(out_dt))
    cp = _chunk_ptrs(chunks)
    rc = _load().oracle_ag_gemm_points(P, Mc, N, K, in_dt, out_dt, cp, _ptr(W), len(ms),
                                       _ptr(ms), _ptr(ns), _ptr(ov))
    if rc != 0:
        raise ValueError(f"oracle_ag_gemm_points rejected its arguments (rc={rc})")
    return ov


def embbag_a2a(T, R, D, B, L, P, tables, indices, offsets=None):
    """Embedding bag + All-to-All.  Returns win [P][B/P][T][D] fp32.
    Raises IndexError if an index lies outside [0, R)."""
    assert tables.dtype == np.float32 and tables.shape == (T, R, D)
    assert indices.dtype == np.int32
    if offsets is not None:
        assert offsets.dtype == np.int64 and offsets.shape == (T * B + 1,)
    win = np.empty((P, B // P, T, D), dtype=np.float32)
    rc = _load().oracle_embbag_a2a(T, R, D, B, L, P, _ptr(tables), _ptr(indices),
                                   _ptr(offsets), _ptr(win))
    if rc == -2:
        raise IndexError("embedding index outside the table")
    if rc != 0:
        raise ValueError(f"oracle_embbag_a2a rejected its arguments (rc={rc})")
    return win
