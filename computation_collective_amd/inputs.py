"""Seeded synthetic inputs for the four fused operators.

This module is shared by the tests, ``bench.py`` and ``smoke()``: it is the
only code that both the CPU oracle and the HIP path consume.  It therefore
holds no arithmetic of the fused operators themselves -- only random draws,
the fp32 -> bf16 encoding of the drawn values (round to nearest even), and
index sampling.

Recipe (the same for every size):

* ``numpy.random.default_rng(seed)`` (PCG64); tensors are drawn in the order
  they are listed for the operator.
* ``N(0, s)``: ``standard_normal(float32) * s`` (``s`` is a standard
  deviation); ``U[-1, 1)``: ``uniform(-1, 1)`` cast to float32.
* bf16 tensors are the round-to-nearest-even encoding of the fp32 draws and
  are carried as ``uint16`` bit patterns.
* Embedding indices: bounded Zipf over ranks ``k = 1..R`` with
  ``p(k) ~ k**-alpha`` and row ``k - 1`` (hot rows are the low row numbers),
  drawn per table by inverse-CDF sampling from
  ``SeedSequence(seed).spawn(T)[t]``.
* Embedding tables too large for host memory are drawn on the device with
  ``torch.randn`` from a ``torch.Generator`` seeded ``seed * 1000 + t`` per
  table (``embbag_tables_torch``); the oracle then receives the rows it needs
  copied back from those same device bytes.
"""

from __future__ import annotations

import numpy as np

F32 = 0
BF16 = 1


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite (the generators never draw NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_decode(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _draw(rng, shape, dist, dtype):
    """Draw one tensor.  dist: ('normal', std) | ('uniform',) | ('int', lo, hi)
    | ('wide', lo, hi): sign * 2**e * (1 + u), e an integer in [lo, hi], u in
    [0, 1) -- magnitudes spread over many binades | ('selector',): a
    [..][rows][cols] 0/1 matrix with a single 1 per row, at column row mod
    cols (drawn from nothing)."""
    kind = dist[0]
    if kind == "normal":
        v = _normal(rng, shape, dist[1])
    elif kind == "uniform":
        v = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    elif kind == "int":
        v = rng.integers(dist[1], dist[2] + 1, size=shape).astype(np.float32)
    elif kind == "wide":
        e = rng.integers(dist[1], dist[2] + 1, size=shape)
        u = rng.uniform(0.0, 1.0, size=shape)
        sign = np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
        v = (sign * np.ldexp(1.0 + u, e)).astype(np.float32)
    elif kind == "selector":
        rows, cols = shape[-2], shape[-1]
        v = np.zeros(shape, dtype=np.float32)
        v[..., np.arange(rows), np.arange(rows) % cols] = 1.0
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return bf16_encode(v) if dtype == BF16 else v


def gemm_rs_inputs(P, M, N, K, dtype, seed=0, dist_a=("normal", 1.0), dist_w=("normal", 0.02)):
    """A [P][M][K] then W [P][K][N]."""
    rng = np.random.default_rng(seed)
    A = _draw(rng, (P, M, K), dist_a, dtype)
    W = _draw(rng, (P, K, N), dist_w, dtype)
    return A, W


def gemv_ar_inputs(P, Mb, N, K, dtype=BF16, seed=0, dist_x=("normal", 1.0), dist_w=("normal", 0.02)):
    """x [P][Mb][K] then W [P][K][N]."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, (P, Mb, K), dist_x, dtype)
    W = _draw(rng, (P, K, N), dist_w, dtype)
    return x, W


def ag_gemm_inputs(P, Mc, N, K, dtype=BF16, seed=0, dist_a=("normal", 1.0), dist_w=("normal", 0.02)):
    """chunks [P][Mc][K], then W [K][N], then the chunk release order."""
    rng = np.random.default_rng(seed)
    chunks = _draw(rng, (P, Mc, K), dist_a, dtype)
    W = _draw(rng, (K, N), dist_w, dtype)
    order = rng.permutation(P).astype(np.int64)
    return chunks, W, order


def zipf_cdf(R: int, alpha: float) -> np.ndarray:
    """CDF of the bounded Zipf law over ranks 1..R (fp64)."""
    w = np.arange(1, R + 1, dtype=np.float64) ** (-alpha)
    c = np.cumsum(w)
    return c / c[-1]


def zipf_indices(T, B, L, R, alpha=1.05, seed=0, cdf=None) -> np.ndarray:
    """int32 indices [T][B][L]; table t drawn from SeedSequence(seed).spawn(T)[t]."""
    if cdf is None:
        cdf = zipf_cdf(R, alpha)
    out = np.empty((T, B, L), dtype=np.int32)
    for t, ss in enumerate(np.random.SeedSequence(seed).spawn(T)):
        u = np.random.default_rng(ss).random(B * L)
        k = np.searchsorted(cdf, u, side="right")
        np.minimum(k, R - 1, out=k)
        out[t] = k.reshape(B, L).astype(np.int32)
    return out


def uniform_indices(T, B, L, R, seed=0) -> np.ndarray:
    out = np.empty((T, B, L), dtype=np.int32)
    for t, ss in enumerate(np.random.SeedSequence(seed).spawn(T)):
        out[t] = np.random.default_rng(ss).integers(0, R, size=(B, L), dtype=np.int32)
    return out


def embbag_tables(T, R, D, std=0.01, seed=0) -> np.ndarray:
    """fp32 tables [T][R][D] drawn on the host (sizes that fit in host memory)."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (T, R, D), std)


def embbag_tables_torch(T, R, D, std=0.01, seed=0, device="cuda"):
    """fp32 tables [T][R][D] drawn on ``device``, one seeded generator per table."""
    import torch

    tab = torch.empty((T, R, D), dtype=torch.float32, device=device)
    for t in range(T):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 1000 + t)
        tab[t].normal_(0.0, 1.0, generator=g)
        tab[t].mul_(std)
    return tab


def tagged_tables(T, R, D) -> np.ndarray:
    """Table t, row i = (i & 0xFFF, i >> 12, t, 1, 0, ...): pooled sums of these
    rows are exact small integers, so a misrouted bag, a wrong index or a wrong
    table shows up bit-exactly (dimension 3 counts the bag's length)."""
    assert D >= 4
    tab = np.zeros((T, R, D), dtype=np.float32)
    i = np.arange(R)
    tab[:, :, 0] = (i & 0xFFF)[None, :]
    tab[:, :, 1] = (i >> 12)[None, :]
    tab[:, :, 2] = np.arange(T, dtype=np.float32)[:, None]
    tab[:, :, 3] = 1.0
    return tab


def csr_bag_offsets(T, B, max_len, seed=0, empty_frac=0.1) -> np.ndarray:
    """int64 offsets [T*B + 1] for ragged bags: lengths uniform in 1..max_len,
    with a fraction ``empty_frac`` of bags forced empty."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, size=T * B)
    lens[rng.random(T * B) < empty_frac] = 0
    off = np.zeros(T * B + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    return off


def moe_choices(P, E, B, topk, seed=0):
    """Top-k router choices of an expert-parallel MoE layer: int32 [P][B][topk],
    source rank p's token b picks `topk` distinct global experts out of the
    P*E, uniformly at random (the first topk of a random permutation)."""
    rng = np.random.default_rng(seed)
    return np.argsort(rng.random((P, B, P * E)), axis=2)[:, :, :topk].astype(np.int32)


def a2a_gemm_inputs(P, B, K, E, N, dtype=BF16, seed=0, dist_x=("normal", 1.0), dist_w=("normal", 0.02)):
    """Token rows X [P][B][K] of the P source ranks, then the local experts'
    weights W [E][K][N]."""
    rng = np.random.default_rng(seed + 1)
    X = _draw(rng, (P, B, K), dist_x, dtype)
    W = _draw(rng, (E, K, N), dist_w, dtype)
    return X, W


def moe_routing(P, E, B, topk, tile_m, seed=0):
    """Top-k routing of an expert-parallel MoE layer, seen from rank 0.

    P ranks each hold B tokens and E experts (P*E experts in all; rank 0 owns
    experts 0..E-1).  Every token picks `topk` distinct experts uniformly at
    random.  Rank 0 computes the pairs (rank d, token t, choice k) whose
    expert is one of its own, grouped by expert, each group in (d, t, k)
    order and padded with empty rows to a multiple of `tile_m` (the
    block-aligned layout of a grouped GEMM).  Each real row goes back to its
    token's rank d, at slot = its position among the pairs rank 0 sends to d,
    in (t, k) order.

    Returns (offsets int64 [E+1] (row ranges of the expert groups), dest int32
    [T] (-1 for a padding row), slot int32 [T] (-1 for padding), send_counts
    int64 [P]), T = offsets[-1]."""
    choice = moe_choices(P, E, B, topk, seed=seed)     # [d][t][k] expert ids
    local = choice < E
    d_idx, t_idx, k_idx = np.nonzero(local)            # (d, t, k) order
    experts = choice[d_idx, t_idx, k_idx]
    send_counts = np.bincount(d_idx, minlength=P).astype(np.int64)
    # slot of each pair inside its destination: running count per d in (t, k) order
    slot_of = np.empty(len(d_idx), dtype=np.int64)
    for d in range(P):
        m = d_idx == d
        slot_of[m] = np.arange(int(m.sum()))
    offsets = np.zeros(E + 1, dtype=np.int64)
    dest_rows, slot_rows = [], []
    for e in range(E):
        m = experts == e
        n = int(m.sum())
        padded = -(-n // tile_m) * tile_m
        dest_e = np.full(padded, -1, dtype=np.int32)
        slot_e = np.full(padded, -1, dtype=np.int32)
        dest_e[:n] = d_idx[m]
        slot_e[:n] = slot_of[m]
        dest_rows.append(dest_e)
        slot_rows.append(slot_e)
        offsets[e + 1] = offsets[e] + padded
    dest = np.concatenate(dest_rows) if dest_rows else np.zeros(0, np.int32)
    slot = np.concatenate(slot_rows) if slot_rows else np.zeros(0, np.int32)
    return offsets, dest, slot, send_counts


def gemm_a2a_inputs(E, T, N, K, dest, dtype=BF16, seed=0, dist_x=("normal", 1.0), dist_w=("normal", 0.02)):
    """X [T][K] (padding rows, dest < 0, are zero) then W [E][K][N]."""
    rng = np.random.default_rng(seed)
    X = _draw(rng, (T, K), dist_x, dtype)
    W = _draw(rng, (E, K, N), dist_w, dtype)
    X[np.asarray(dest) < 0] = 0
    return X, W
