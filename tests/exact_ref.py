"""Brute-force exact reference for tiny cases, used to pin the CPU oracle.

Written independently of the oracle: Python rationals (``fractions.Fraction``)
carry every sum exactly, and rounding to binary32 / bfloat16 is implemented
here from the IEEE-754 definition (round to nearest, ties to even, gradual
underflow).  Only for inputs of a few elements per dimension.

Semantics restated from the pages: "Optimizing Distributed ML Communication
with Fused Computation-Collective Operations" (SC24, abstract) fuses each
computation with its subsequent collective; the result is that of the
computation followed by the collective.  Readings where the pages are silent:
partials are fp32-rounded exact dot products (then bf16-rounded when carried
in bf16), reduced by an fp32 left fold in rank order, rounded once to the
output type.
"""

from fractions import Fraction
import math

FP32 = (24, -126, 127)   # significand bits (with the hidden bit), emin, emax
BF16 = (8, -126, 127)


def _exponent(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2**e <= a < 2**(e+1) after at most one correction either way
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to(x: Fraction, fmt) -> Fraction:
    """Round x to the binary format fmt, nearest with ties to even.
    Returns a Fraction, or +-inf as a float when the result overflows."""
    p, emin, emax = fmt
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_exponent(a), emin)          # below emin the quantum stops shrinking
    q = Fraction(2) ** (e - p + 1)        # spacing of representable values here
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    if r >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * r


def fr(v) -> Fraction:
    return Fraction(float(v))


def gemm_rs(P, M, N, K, A, W, slot_fmt, out_fmt):
    """A, W nested lists of numbers.  Returns (slots[r][p][i][n], out[m][n]) as Fractions."""
    assert M % P == 0
    Mc = M // P
    C = [[[None] * N for _ in range(M)] for _ in range(P)]
    for p in range(P):
        for m in range(M):
            for n in range(N):
                s = sum((fr(A[p][m][k]) * fr(W[p][k][n]) for k in range(K)), Fraction(0))
                c = round_to(s, FP32)
                if slot_fmt is BF16:
                    c = round_to(c, BF16)
                C[p][m][n] = c
    slots = [[[[C[p][r * Mc + i][n] for n in range(N)] for i in range(Mc)] for p in range(P)]
             for r in range(P)]
    out = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = C[0][m][n]
            for p in range(1, P):
                acc = round_to(acc + C[p][m][n], FP32)
            out[m][n] = round_to(acc, out_fmt) if out_fmt is BF16 else acc
    return slots, out


def gemm_ar(P, M, N, K, A, W, slot_fmt, out_fmt):
    """Returns (slots[r][p][i][n], win[q][m][n]): every window q holds the full
    rank-order sum (the reduced chunks gathered in destination order)."""
    slots, out = gemm_rs(P, M, N, K, A, W, slot_fmt, out_fmt)
    return slots, [[list(out[m]) for m in range(M)] for _ in range(P)]


def gemm_a2a(P, E, N, K, X, W, offsets, dest, slot, cap, out_fmt):
    """Returns win[d][s][n] (None where no row lands) as Fractions."""
    win = [[[None] * N for _ in range(cap)] for _ in range(P)]
    for e in range(E):
        for i in range(offsets[e], offsets[e + 1]):
            if dest[i] < 0:
                continue
            for n in range(N):
                s = sum((fr(X[i][k]) * fr(W[e][k][n]) for k in range(K)), Fraction(0))
                v = round_to(s, FP32)
                win[dest[i]][slot[i]][n] = round_to(v, out_fmt) if out_fmt is BF16 else v
    return win


def a2a_gemm(P, E, e0, B, topk, N, K, X, experts, W, tile_m, out_fmt):
    """MoE dispatch + GEMM by enumeration: for each local expert, the pairs
    (p, b, j) that chose it, listed in (p, b, j) order; the group padded to a
    multiple of tile_m; a pair's slot = its index in the list of its source's
    pairs that choose any local expert.  Returns (rows, offsets, send_counts)
    with rows[i] = (dest, slot, token row as a list, Y row as Fractions); a
    padding row is (-1, -1, None, zeros)."""
    local = lambda v: e0 <= v < e0 + E
    per_source = [[(b, j) for b in range(B) for j in range(topk) if local(experts[p][b][j])] for p in range(P)]
    rows, offsets = [], [0]
    for e in range(E):
        pairs = [(p, b, j) for p in range(P) for b in range(B) for j in range(topk) if experts[p][b][j] == e0 + e]
        for (p, b, j) in pairs:
            y = []
            for n in range(N):
                s = sum((fr(X[p][b][k]) * fr(W[e][k][n]) for k in range(K)), Fraction(0))
                v = round_to(s, FP32)
                y.append(round_to(v, out_fmt) if out_fmt is BF16 else v)
            rows.append((p, per_source[p].index((b, j)), list(X[p][b]), y))
        pad = -len(pairs) % tile_m
        rows += [(-1, -1, None, [Fraction(0)] * N)] * pad
        offsets.append(offsets[-1] + len(pairs) + pad)
    return rows, offsets, [len(per_source[p]) for p in range(P)]


def gemv_ar(P, Mb, N, K, x, W, slot_fmt, out_fmt):
    """Returns (part[p][b][n], win[q][b][n])."""
    part = [[[None] * N for _ in range(Mb)] for _ in range(P)]
    for p in range(P):
        for b in range(Mb):
            for n in range(N):
                s = sum((fr(x[p][b][k]) * fr(W[p][k][n]) for k in range(K)), Fraction(0))
                c = round_to(s, FP32)
                if slot_fmt is BF16:
                    c = round_to(c, BF16)
                part[p][b][n] = c
    res = [[None] * N for _ in range(Mb)]
    for b in range(Mb):
        for n in range(N):
            acc = part[0][b][n]
            for p in range(1, P):
                acc = round_to(acc + part[p][b][n], FP32)
            res[b][n] = round_to(acc, out_fmt) if out_fmt is BF16 else acc
    win = [[list(res[b]) for b in range(Mb)] for _ in range(P)]
    return part, win


def ag_gemm(P, Mc, N, K, chunks, W, out_fmt):
    """chunks[c][i][k]; returns (gathered[m][k], out[m][n])."""
    gathered = [row for c in range(P) for row in chunks[c]]
    out = []
    for m in range(P * Mc):
        row = []
        for n in range(N):
            s = sum((fr(gathered[m][k]) * fr(W[k][n]) for k in range(K)), Fraction(0))
            v = round_to(s, FP32)
            if out_fmt is BF16:
                v = round_to(v, BF16)
            row.append(v)
        out.append(row)
    return gathered, out


def embbag_a2a(T, R, D, B, P, tables, bags):
    """bags[t][b] = list of row indices.  Returns win[d][s][t][:] as Fractions."""
    Bd = B // P
    win = [[[None for _ in range(T)] for _ in range(Bd)] for _ in range(P)]
    for t in range(T):
        for b in range(B):
            acc = [Fraction(0)] * D
            for row in bags[t][b]:
                acc = [round_to(acc[d] + fr(tables[t][row][d]), FP32) for d in range(D)]
            win[b // Bd][b % Bd][t] = acc
    return win
