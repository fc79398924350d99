"""Device buffers for one call of each fused operator, and the call itself.

Owns the plumbing around an entry point -- uploading the seeded inputs,
allocating the receive windows, flag arrays, workspace and status word with
PyTorch, advancing the epoch -- so that tests, the bench and the smoke check
drive the C ABI the same way.  No arithmetic of the operators lives here.
bf16 tensors are carried as ``torch.int16`` (their bit patterns).
"""

from __future__ import annotations

import numpy as np
import torch

from . import hocf

F32, BF16 = hocf.HOCF_F32, hocf.HOCF_BF16


def tdtype(dt):
    return torch.int16 if dt == BF16 else torch.float32


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor, dt) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if dt == BF16 else a


def nan_fill(t: torch.Tensor) -> None:
    """Poison a buffer so that any element the kernel does not write shows up."""
    if t.dtype == torch.int16:
        t.fill_(0x7FC0)          # bf16 quiet NaN
    elif t.dtype == torch.float32:
        t.fill_(float("nan"))
    else:
        t.fill_(-1)


def cdiv(a, b):
    return (a + b - 1) // b


class _Common:
    def _alloc_sync(self, ws_bytes, device):
        self.ws_bytes = max(int(ws_bytes), 16)
        self.ws = torch.zeros(cdiv(self.ws_bytes, 4) + 4, dtype=torch.int32, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.epoch = 0

    def next_sync(self, spin_timeout_ns=0, abort_flag=None):
        self.epoch = (self.epoch % 0xFFFFFFF0) + 1
        return hocf.sync(self.epoch, self.ws, self.ws_bytes, status=self.status,
                         abort_flag=abort_flag, spin_timeout_ns=spin_timeout_ns)

    def status_value(self) -> int:
        return int(self.status.item())


class GemmRS(_Common):
    """hocf_gemm_rs: A [P][M][K], W [P][K][N] -> windows [P dst][P src][Mc][N], out [M][N]."""

    def __init__(self, P, M, N, K, in_dt, slot_dt, out_dt, tile_m, tile_n, A, W, device="cuda",
                 unfused=False, noalloc=False, pieces=0, fold_cus=0):
        self.unfused = unfused   # hocf_gemm_rs_unfused: the GEMM kernel, then the fold kernel
        self.noalloc = noalloc   # hocf_gemm_rs_noalloc: no workspace (the library's scratch)
        # hocf_gemm_rs_decomposed: `pieces` column pieces, GEMM on the call's stream (leaving
        # fold_cus CUs), each fold on a second stream
        self.pieces, self.fold_cus = pieces, fold_cus
        self.coll = torch.cuda.Stream(device=device) if pieces else None
        self.P, self.M, self.N, self.K = P, M, N, K
        self.in_dt, self.slot_dt, self.out_dt = in_dt, slot_dt, out_dt
        self.tile_m, self.tile_n = tile_m, tile_n
        self.Mc = M // P
        self.A = A if isinstance(A, torch.Tensor) else to_device(A, device)
        self.W = W if isinstance(W, torch.Tensor) else to_device(W, device)
        self.tpc = cdiv(self.Mc, tile_m) * cdiv(N, tile_n)
        self.win_data = torch.empty((P, P, self.Mc, N), dtype=tdtype(slot_dt), device=device)
        self.win_flags = torch.zeros((P, P, self.tpc), dtype=torch.int32, device=device)
        self.out = torch.empty((M, N), dtype=tdtype(out_dt), device=device)
        self.win = hocf.windows([(self.win_data[r], self.win_flags[r]) for r in range(P)])
        self._alloc_sync(hocf.hocf_gemm_rs_workspace_bytes(P, M, N, tile_m, tile_n), device)

    def poison(self):
        nan_fill(self.win_data)
        nan_fill(self.out)

    def call(self, stream=None, **kw) -> int:
        s = self.next_sync(**kw)
        if getattr(self, "pieces", 0):
            return hocf.hocf_gemm_rs_decomposed(self.P, self.M, self.N, self.K, self.in_dt, self.slot_dt,
                                                self.out_dt, self.A, self.W, self.win, self.out, self.tile_m,
                                                self.tile_n, self.pieces, self.fold_cus, s,
                                                stream if stream is not None else torch.cuda.current_stream(),
                                                self.coll)
        if getattr(self, "noalloc", False):
            s.workspace, s.workspace_bytes = None, 0
            fn = hocf.hocf_gemm_rs_noalloc
        else:
            fn = hocf.hocf_gemm_rs_unfused if self.unfused else hocf.hocf_gemm_rs
        return fn(self.P, self.M, self.N, self.K, self.in_dt, self.slot_dt, self.out_dt, self.A, self.W,
                  self.win, self.out, self.tile_m, self.tile_n, s, stream)

    def run(self, stream=None, **kw):
        hocf.check(self.call(stream, **kw))


class GemmAR(GemmRS):
    """hocf_gemm_ar: as GemmRS, and every destination q gets the whole reduced
    result in outs[q] = [M][N] (held together as out_all [P][M][N])."""

    def __init__(self, P, M, N, K, in_dt, slot_dt, out_dt, tile_m, tile_n, A, W, device="cuda"):
        super().__init__(P, M, N, K, in_dt, slot_dt, out_dt, tile_m, tile_n, A, W, device)
        del self.unfused
        del self.out
        self.out_all = torch.empty((P, M, N), dtype=tdtype(out_dt), device=device)
        self.outs = hocf.pointers([self.out_all[q] for q in range(P)])

    def poison(self):
        nan_fill(self.win_data)
        nan_fill(self.out_all)

    def call(self, stream=None, **kw) -> int:
        s = self.next_sync(**kw)
        return hocf.hocf_gemm_ar(self.P, self.M, self.N, self.K, self.in_dt, self.slot_dt,
                                 self.out_dt, self.A, self.W, self.win, self.outs, self.tile_m,
                                 self.tile_n, s, stream)


class GemvAR(_Common):
    """hocf_gemv_ar: x [P][Mb][K], W [P][K][N] -> part [P][Mb][N], windows [P][Mb][N]."""

    def __init__(self, P, Mb, N, K, in_dt, slot_dt, out_dt, tile_n, x, W, device="cuda", unfused=False):
        self.unfused = unfused   # hocf_gemv_ar_unfused: the GEMV kernel, then the fold kernel
        self.P, self.Mb, self.N, self.K = P, Mb, N, K
        self.in_dt, self.slot_dt, self.out_dt, self.tile_n = in_dt, slot_dt, out_dt, tile_n
        self.x = x if isinstance(x, torch.Tensor) else to_device(x, device)
        self.W = W if isinstance(W, torch.Tensor) else to_device(W, device)
        self.nt = cdiv(N, tile_n)
        self.part = torch.empty((P, Mb, N), dtype=tdtype(slot_dt), device=device)
        self.part_flags = torch.zeros((P, self.nt), dtype=torch.int32, device=device)
        self.win_data = torch.empty((P, Mb, N), dtype=tdtype(out_dt), device=device)
        self.win_flags = torch.zeros((P, self.nt), dtype=torch.int32, device=device)
        self.win = hocf.windows([(self.win_data[q], self.win_flags[q]) for q in range(P)])
        self._alloc_sync(hocf.hocf_gemv_ar_workspace_bytes(P, N, tile_n), device)

    def set_weights(self, x, W):
        self.x, self.W = x, W

    def poison(self):
        nan_fill(self.part)
        nan_fill(self.win_data)

    def call(self, stream=None, **kw) -> int:
        s = self.next_sync(**kw)
        fn = hocf.hocf_gemv_ar_unfused if self.unfused else hocf.hocf_gemv_ar
        return fn(self.P, self.Mb, self.N, self.K, self.in_dt, self.slot_dt, self.out_dt, self.x, self.W,
                  self.part, self.part_flags, self.win, self.tile_n, s, stream)

    def run(self, stream=None, **kw):
        hocf.check(self.call(stream, **kw))


class AgGemm(_Common):
    """hocf_ag_gemm: gathered chunks [P][Mc][K] gated by chunk_flags [P]; W [K][N] -> out.

    flags="device": chunk flags in device memory, written on the kernel's own
    stream before the kernel (all chunks present when it starts).
    flags="host": chunk flags in coherent pinned host memory, written by the
    host while the kernel runs (paced, any order, or withheld).
    chunks_on_host: the gathered chunks themselves live in coherent pinned host
    memory too, so the host can deliver them after the kernel has started."""

    def __init__(self, P, Mc, N, K, out_dt, tile_m, tile_n, chunks, W, device="cuda",
                 flags="device", chunks_on_host=False):
        self.P, self.Mc, self.N, self.K = P, Mc, N, K
        self.out_dt, self.tile_m, self.tile_n = out_dt, tile_m, tile_n
        self.flags_mode = flags
        self.W = W if isinstance(W, torch.Tensor) else to_device(W, device)
        self.host_chunks = None
        if chunks_on_host:
            nbytes = P * Mc * K * 2
            addr, _ = hocf.host_coherent(nbytes)
            self.A = addr
            self.host_chunks = np.frombuffer((ctypes_char_array(addr, nbytes)), dtype=np.uint16).reshape(P, Mc, K)
        else:
            self.A = chunks if isinstance(chunks, torch.Tensor) else to_device(chunks, device)
        if flags == "host":
            addr, _ = hocf.host_coherent(4 * P)
            self.chunk_flags = addr
            self.host_flags = np.frombuffer(ctypes_char_array(addr, 4 * P), dtype=np.uint32)
        else:
            self.chunk_flags = torch.zeros(P, dtype=torch.int32, device=device)
            self.host_flags = None
        self.out = torch.empty((P * Mc, N), dtype=tdtype(out_dt), device=device)
        self._alloc_sync(hocf.hocf_ag_gemm_workspace_bytes(P), device)

    def poison(self):
        nan_fill(self.out)

    def call(self, sync_, stream=None) -> int:
        return hocf.hocf_ag_gemm(self.P, self.Mc, self.N, self.K, BF16, self.out_dt, self.A,
                                 self.chunk_flags, self.W, self.out, self.tile_m, self.tile_n,
                                 sync_, stream)

    def prerelease(self, order, stream=None, **kw):
        """Writes the chunk flags in `order` on `stream` for the next call; returns its sync."""
        assert self.flags_mode == "device"
        s = self.next_sync(**kw)
        hocf.release_chunks(stream or torch.cuda.current_stream(), self.chunk_flags, order, s.epoch)
        return s

    def launch(self, sync_, stream=None):
        hocf.check(self.call(sync_, stream or torch.cuda.current_stream()))

    def run_prereleased(self, order, stream=None, **kw):
        """Flags written in `order` on the kernel's stream, then the kernel."""
        stream = stream or torch.cuda.current_stream()
        self.launch(self.prerelease(order, stream, **kw), stream)

    def run_host_released(self, order, delay_s=0.0, deliver=None, stream=None, **kw):
        """Kernel first; then the host sets the flags of `order` one by one (after
        `delay_s` each), optionally delivering chunk c's data first via deliver(c)."""
        import time
        assert self.flags_mode == "host"
        s = self.next_sync(**kw)
        stream = stream or torch.cuda.current_stream()
        hocf.check(self.call(s, stream))
        for c in order:
            if delay_s:
                time.sleep(delay_s)
            if deliver is not None:
                deliver(int(c))
            self.host_flags[int(c)] = s.epoch
        return s.epoch


    def put_delivered(self, sources, order, engine, put_stream, stream=None, **kw):
        """Chunks delivered by hocf_dma_put on `put_stream` while the kernel runs on
        `stream`: one put per chunk in `order` (chunk c's bytes from sources[c] into
        its rows of the gathered buffer, then its flag); sources[c] None: the chunk is
        already in place (the local one) and its put only signals.  The puts are
        enqueued first and wait for nothing but `stream`'s earlier work, so the
        kernel starts while they land.  Returns the call's sync."""
        assert self.flags_mode == "device" and isinstance(self.A, torch.Tensor)
        stream = stream or torch.cuda.current_stream()
        s = self.next_sync(**kw)
        if s.epoch >= _EPOCH_WORDS:
            # the signal table holds epochs below 2^16: start over at 1 (it still
            # differs from the previous call's epoch, the flags' only requirement)
            self.epoch = 0
            s = self.next_sync(**kw)
        chunk_bytes = self.Mc * self.K * 2
        base, fbase = self.A.data_ptr(), self.chunk_flags.data_ptr()
        src, dst, nbytes, sig = [], [], [], []
        for c in order:
            c = int(c)
            here = sources[c] is None
            src.append(None if here else sources[c])
            dst.append(None if here else base + c * chunk_bytes)
            nbytes.append(0 if here else chunk_bytes)
            sig.append(fbase + 4 * c)
        put_stream.wait_stream(stream)
        hocf.check(hocf.hocf_dma_put(src, dst, nbytes, sig, epoch_word(s.epoch, self.A.device), engine,
                                     put_stream))
        hocf.check(self.call(s, stream))
        stream.wait_stream(put_stream)
        return s


_epoch_words = {}
_EPOCH_WORDS = 1 << 16


def epoch_word(epoch: int, device) -> int:
    """Device address of a word holding `epoch` (1 <= epoch < 65536), from a table
    written once per device: the source a put copies into a flag, so that the
    put's signal needs no kernel to prepare it."""
    assert 1 <= epoch < _EPOCH_WORDS, epoch
    key = str(device)
    if key not in _epoch_words:
        _epoch_words[key] = torch.arange(_EPOCH_WORDS, dtype=torch.int32, device=device)
        torch.cuda.synchronize(device)
    return _epoch_words[key].data_ptr() + 4 * epoch


def ctypes_char_array(addr, nbytes):
    import ctypes
    return (ctypes.c_char * nbytes).from_address(addr)


class EmbbagA2A(_Common):
    """hocf_embbag_a2a: tables [T][R][D], indices -> windows [P][Bd][T][D]."""

    def __init__(self, T, R, D, B, L, P, tile_bags, tables, indices, offsets=None, device="cuda"):
        self.T, self.R, self.D, self.B, self.L, self.P = T, R, D, B, L, P
        self.tile_bags = tile_bags
        self.Bd = B // P
        self.nj = cdiv(self.Bd, tile_bags)
        self.tables = tables if isinstance(tables, torch.Tensor) else to_device(tables, device)
        self.indices = indices if isinstance(indices, torch.Tensor) else to_device(indices, device)
        self.offsets = None
        if offsets is not None:
            self.offsets = offsets if isinstance(offsets, torch.Tensor) else to_device(offsets, device)
        self.win_data = torch.empty((P, self.Bd, T, D), dtype=torch.float32, device=device)
        self.win_flags = torch.zeros((P, T, self.nj), dtype=torch.int32, device=device)
        self.win = hocf.windows([(self.win_data[d], self.win_flags[d]) for d in range(P)])
        self._alloc_sync(hocf.hocf_embbag_a2a_workspace_bytes(), device)

    def poison(self):
        nan_fill(self.win_data)

    def call(self, stream=None, **kw) -> int:
        s = self.next_sync(**kw)
        return hocf.hocf_embbag_a2a(self.T, self.R, self.D, self.B, 0 if self.offsets is not None else self.L,
                                    self.P, self.tables, self.indices, self.offsets, self.win,
                                    self.tile_bags, s, stream)

    def run(self, stream=None, **kw):
        hocf.check(self.call(stream, **kw))


class GemmA2A(_Common):
    """hocf_gemm_a2a: X [T][K] grouped by expert (offsets), W [E][K][N], routing
    dest/slot [T] -> windows [P][cap][N] with one flag word each."""

    def __init__(self, P, E, N, K, out_dt, X, W, offsets, dest, slot, send_counts, cap, device="cuda",
                 tile_m=256):
        self.P, self.E, self.N, self.K, self.out_dt, self.cap = P, E, N, K, out_dt, cap
        self.tile_m = tile_m
        self.offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        self.send_counts = np.ascontiguousarray(send_counts, dtype=np.int64)
        self.T = int(self.offsets[-1])
        self.X = X if isinstance(X, torch.Tensor) else to_device(X, device)
        self.W = W if isinstance(W, torch.Tensor) else to_device(W, device)
        self.dest = to_device(np.ascontiguousarray(dest, dtype=np.int32), device)
        self.slot = to_device(np.ascontiguousarray(slot, dtype=np.int32), device)
        self.win_data = torch.empty((P, cap, N), dtype=tdtype(out_dt), device=device)
        self.win_flags = torch.zeros((P, 4), dtype=torch.int32, device=device)  # word 0 used; 16-byte rows
        self.win = hocf.windows([(self.win_data[d], self.win_flags[d]) for d in range(P)])
        self._alloc_sync(hocf.hocf_gemm_a2a_workspace_bytes(P), device)

    def poison(self):
        nan_fill(self.win_data)

    def call(self, stream=None, **kw) -> int:
        s = self.next_sync(**kw)
        return hocf.hocf_gemm_a2a(self.P, self.E, self.T, self.N, self.K, BF16, self.out_dt, self.X, self.W,
                                  self.offsets, self.dest, self.slot, self.send_counts, self.win, self.cap,
                                  self.tile_m, 256, s, stream)

    def run(self, stream=None, **kw):
        hocf.check(self.call(stream, **kw))


class A2aGemm(_Common):
    """hocf_a2a_gemm: token rows X [P][B][K] and router choices [P][B][topk] of the
    P source ranks, this rank's experts W [E][K][N] (global ids e0 ..) -> the
    received rows recv [cap][K] grouped by expert, Y [cap][N], expert_offsets
    [E+1], dest / slot [cap], send_counts [P]."""

    def __init__(self, P, E, e0, B, topk, N, K, out_dt, X, experts, W, cap, tile_m=256, device="cuda",
                 unfused=False):
        self.P, self.E, self.e0, self.B, self.topk, self.N, self.K = P, E, e0, B, topk, N, K
        self.out_dt, self.cap, self.tile_m, self.unfused = out_dt, cap, tile_m, unfused
        self.X = X if isinstance(X, torch.Tensor) else to_device(X, device)
        self.W = W if isinstance(W, torch.Tensor) else to_device(W, device)
        self.experts = experts if isinstance(experts, torch.Tensor) else \
            to_device(np.ascontiguousarray(experts, dtype=np.int32), device)
        self.recv = torch.empty((cap, K), dtype=torch.int16, device=device)
        self.Y = torch.empty((cap, N), dtype=tdtype(out_dt), device=device)
        self.offsets = torch.empty(E + 1, dtype=torch.int64, device=device)
        self.dest = torch.empty(cap, dtype=torch.int32, device=device)
        self.slot = torch.empty(cap, dtype=torch.int32, device=device)
        self.send_counts = torch.empty(P, dtype=torch.int64, device=device)
        self._alloc_sync(hocf.hocf_a2a_gemm_workspace_bytes(P, E, B, topk, cap, tile_m), device)

    def poison(self):
        nan_fill(self.recv)
        nan_fill(self.Y)
        self.dest.fill_(-77)        # (not -1: that is what padding rows get)
        self.slot.fill_(-77)
        self.offsets.fill_(-7)
        self.send_counts.fill_(-7)

    def call(self, stream=None, **kw) -> int:
        s = self.next_sync(**kw)
        return hocf.hocf_a2a_gemm(self.P, self.E, self.e0, self.B, self.topk, self.N, self.K, BF16, self.out_dt,
                                  self.X, self.experts, self.W, self.cap, self.recv, self.Y, self.offsets,
                                  self.dest, self.slot, self.send_counts, self.tile_m, 256, s, stream,
                                  unfused=self.unfused)

    def run(self, stream=None, **kw):
        hocf.check(self.call(stream, **kw))
