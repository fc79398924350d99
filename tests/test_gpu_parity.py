"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Values: normwise relative error <= 2e-2 for bf16 inputs with fp32
accumulation, <= 1e-5 for fp32; integer-valued inputs, routing, indices,
flags and the embedding sums: bit-exact.  Small cases span several tiles and
a ragged tail in every dimension; the full-size workloads run in the launch
configuration the bench times and are compared on sampled outputs plus
properties that hold at any size.  Every output buffer is NaN-poisoned first,
so an element the kernels fail to write cannot pass.
"""

import numpy as np
import pytest
import torch

import oracle
from computation_collective_amd import buffers as bf
from computation_collective_amd import configs as cfgs
from computation_collective_amd import hocf
from computation_collective_amd import inputs as gen

pytestmark = pytest.mark.gpu
F32, BF16 = 0, 1
TOL = {F32: 1e-5, BF16: 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def val(a, dt):
    return (gen.bf16_decode(a) if dt == BF16 else a).astype(np.float64)


def relerr(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert not np.isnan(g).any(), "unwritten (NaN) elements"
    return float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-30))


def sync():
    torch.cuda.synchronize()


# ====================================================================== GEMM + RS

def _gemm_rs(P, Mc, N, K, in_dt, slot_dt, out_dt, tm, tn, seed=0, dist=None):
    M = P * Mc
    if dist is None:
        dist = dict(dist_a=("normal", 1.0), dist_w=("normal", 0.02)) if in_dt == BF16 else \
            dict(dist_a=("uniform",), dist_w=("uniform",))
    A, W = gen.gemm_rs_inputs(P, M, N, K, in_dt, seed=seed, **dist)
    run = bf.GemmRS(P, M, N, K, in_dt, slot_dt, out_dt, tm, tn, A, W)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    slots, out = oracle.gemm_rs(P, M, N, K, in_dt, slot_dt, out_dt, A, W)
    return run, slots, out


def test_gemm_rs_tiny_config():
    c = cfgs.GEMM_RS_TINY
    say(f"gemm_rs {c.name}")
    run, slots, out = _gemm_rs(c.P, c.M // c.P, c.N, c.K, F32, F32, F32, c.tile_m, c.tile_n)
    assert relerr(bf.to_host(run.out, F32), out) <= TOL[F32]
    assert relerr(bf.to_host(run.win_data, F32), slots) <= TOL[F32]
    assert torch.all(run.win_flags == run.epoch)
    assert torch.all(run.ws == 0), "workspace must be left zeroed"


RAGGED = [
    (3, 100, 200, 76, F32, F32, F32, 64, 64),
    (4, 300, 328, 136, BF16, F32, BF16, 256, 256),
    (4, 300, 328, 136, BF16, BF16, BF16, 256, 256),
    (3, 300, 328, 136, BF16, F32, F32, 128, 128),
    (3, 300, 328, 136, BF16, BF16, F32, 128, 128),
    (2, 513, 1032, 72, BF16, F32, BF16, 256, 256),
]


@pytest.mark.parametrize("P,Mc,N,K,ind,sdt,odt,tm,tn", RAGGED)
def test_gemm_rs_ragged(P, Mc, N, K, ind, sdt, odt, tm, tn):
    say(f"gemm_rs ragged P={P} Mc={Mc} N={N} K={K} dt={ind}{sdt}{odt} tile={tm}x{tn}")
    run, slots, out = _gemm_rs(P, Mc, N, K, ind, sdt, odt, tm, tn, seed=P + K)
    assert relerr(val(bf.to_host(run.out, odt), odt), val(out, odt)) <= TOL[ind]
    assert relerr(val(bf.to_host(run.win_data, sdt), sdt), val(slots, sdt)) <= TOL[ind]
    assert torch.all(run.win_flags == run.epoch)
    assert torch.all(run.ws == 0)


@pytest.mark.parametrize("sdt,odt,tm", [(F32, BF16, 256), (BF16, BF16, 256), (F32, F32, 128)])
def test_gemm_rs_integer_bit_exact(sdt, odt, tm):
    """Entries in {-2..2}: every partial and fold is an exact integer, so the HIP
    result equals the oracle bit for bit (bf16 rounding included)."""
    say(f"gemm_rs integer P=4 Mc=300 N=328 K=392 slot={sdt} out={odt} tile={tm}")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run, slots, out = _gemm_rs(4, 300, 328, 392, BF16, sdt, odt, tm, tm, seed=9, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.out, odt), out)
    np.testing.assert_array_equal(bf.to_host(run.win_data, sdt), slots)


@pytest.mark.parametrize("tm,sdt,odt", [(256, F32, BF16), (256, BF16, BF16), (128, F32, F32), (128, BF16, BF16)])
def test_gemm_rs_full_tiles_integer_bit_exact(tm, sdt, odt):
    """Full tiles with K a multiple of 128 take the direct-to-LDS mainloop
    (transposing LDS reads); integer inputs make it bit-exact."""
    P, Mc, N, K = 3, 2 * tm, 2 * tm, 384
    say(f"gemm_rs full tiles integer P={P} Mc={Mc} N={N} K={K} tile={tm} slot={sdt} out={odt}")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run, slots, out = _gemm_rs(P, Mc, N, K, BF16, sdt, odt, tm, tm, seed=tm + sdt, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.out, odt), out)
    np.testing.assert_array_equal(bf.to_host(run.win_data, sdt), slots)


@pytest.mark.parametrize("K,tm,sdt", [(192, 256, F32), (320, 256, BF16), (1856, 256, F32), (448, 128, F32)])
def test_gemm_rs_full_tiles_k_not_whole_rounds_integer_bit_exact(K, tm, sdt):
    """Full row and column tiles with K = 64 (mod 128): the direct-to-LDS
    mainloop covers only K in whole rounds of 128, so the launcher must send
    these to the register-staged mainloop (bit-exact on integer inputs)."""
    P, Mc, N = 3, 2 * tm, 2 * tm
    say(f"gemm_rs full tiles, K={K} (not a multiple of 128), integer, tile={tm} slot={sdt}")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run, slots, out = _gemm_rs(P, Mc, N, K, BF16, sdt, BF16, tm, tm, seed=K, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.out, BF16), out)
    np.testing.assert_array_equal(bf.to_host(run.win_data, sdt), slots)


@pytest.mark.parametrize("op", ["gemm_rs", "gemv_ar"])
def test_abort_word_set_before_the_call(op):
    """With the abort word already nonzero, every wait of the call ends at once
    (HOCF_ERR_ABORTED) and the kernel exits; a call that happened not to wait
    reports OK, and its result is then right (integer inputs: bit-exact)."""
    say(f"{op} with the abort word set before the call")
    addr, _ = hocf.host_coherent(4)
    np.frombuffer(bf.ctypes_char_array(addr, 4), dtype=np.uint32)[0] = 1
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    if op == "gemm_rs":
        P, Mc, N, K = 4, 512, 512, 256
        A, W = gen.gemm_rs_inputs(P, P * Mc, N, K, BF16, seed=21, **ints)
        run = bf.GemmRS(P, P * Mc, N, K, BF16, F32, BF16, 256, 256, A, W)
        _, want = oracle.gemm_rs(P, P * Mc, N, K, BF16, F32, BF16, A, W, want_slots=False)
        got = lambda: bf.to_host(run.out, BF16)
    else:
        P, Mb, N, K = 8, 4, 1024, 512
        x, W = gen.gemv_ar_inputs(P, Mb, N, K, seed=21, dist_x=("int", -2, 2), dist_w=("int", -2, 2))
        run = bf.GemvAR(P, Mb, N, K, BF16, F32, BF16, 256, x, W)
        _, want = oracle.gemv_ar(P, Mb, N, K, BF16, F32, BF16, x, W)
        got = lambda: bf.to_host(run.win_data, BF16)
    for _ in range(3):
        run.status.zero_()
        run.poison()
        run.run(abort_flag=addr, spin_timeout_ns=5_000_000_000)
        sync()
        st = run.status_value()
        assert st in (0, hocf.HOCF_ERR_ABORTED)
        if st == 0:
            np.testing.assert_array_equal(got(), want)
        assert torch.all(run.ws == 0), "the call must leave the workspace zeroed"


@pytest.mark.parametrize("tm", [256, 128])
def test_gemm_rs_full_tiles_values(tm):
    P, Mc, N, K = 4, 2 * tm, 3 * tm, 512
    say(f"gemm_rs full tiles N(0,1) P={P} Mc={Mc} N={N} K={K} tile={tm}")
    run, slots, out = _gemm_rs(P, Mc, N, K, BF16, F32, BF16, tm, tm, seed=tm)
    assert relerr(val(bf.to_host(run.out, BF16), BF16), val(out, BF16)) <= TOL[BF16]
    assert relerr(bf.to_host(run.win_data, F32), slots) <= TOL[BF16]
    assert torch.all(run.win_flags == run.epoch)


def test_gemm_rs_fp32_integer_bit_exact():
    say("gemm_rs fp32 integer P=4 256x256x256 tile 64")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run, slots, out = _gemm_rs(4, 64, 256, 256, F32, F32, F32, 64, 64, seed=3, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.out, F32), out)


def test_gemm_rs_run_to_run_identical():
    say("gemm_rs determinism: 50 calls on one buffer set, bit-identical")
    P, Mc, N, K = 4, 512, 512, 256
    A, W = gen.gemm_rs_inputs(P, P * Mc, N, K, BF16, seed=1)
    run = bf.GemmRS(P, P * Mc, N, K, BF16, F32, BF16, 256, 256, A, W)
    run.run()
    sync()
    ref = run.out.clone()
    for _ in range(50):
        run.poison()
        run.run()
    sync()
    assert torch.equal(run.out, ref)
    assert run.status_value() == 0


@pytest.mark.parametrize("sdt", [F32, BF16])
def test_gemm_rs_alternating_inputs_no_stale_reads(sdt):
    """Two integer input sets alternate on one buffer set with nothing cleared
    between calls: a reducer that read a slot before its producer's stores
    were visible would fold the previous call's (different) partial and miss
    the bit-exact result."""
    P, Mc, N, K = 8, 512, 512, 256
    say(f"gemm_rs alternating inputs P={P} Mc={Mc} N={N} K={K} slot={sdt}")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    sets = []
    for seed in (21, 22):
        A, W = gen.gemm_rs_inputs(P, P * Mc, N, K, BF16, seed=seed, **ints)
        slots, out = oracle.gemm_rs(P, P * Mc, N, K, BF16, sdt, BF16, A, W)
        sets.append((bf.to_device(A), bf.to_device(W), slots, out))
    run = bf.GemmRS(P, P * Mc, N, K, BF16, sdt, BF16, 256, 256, sets[0][0], sets[0][1])
    for call in range(8):
        A, W, slots, out = sets[call % 2]
        run.A, run.W = A, W
        run.run()
        sync()
        assert run.status_value() == 0
        np.testing.assert_array_equal(bf.to_host(run.out, BF16), out, err_msg=f"call {call}")
        np.testing.assert_array_equal(bf.to_host(run.win_data, sdt), slots, err_msg=f"call {call}")


@pytest.mark.parametrize("P,tm,sdt", [(4, 256, F32), (8, 256, F32), (4, 256, BF16), (3, 128, F32)])
def test_gemm_rs_band_in_mainloop_integer_bit_exact(P, tm, sdt, monkeypatch):
    """A small grid makes every workgroup take several tiles, so the bands of
    completed tiles are folded during later tiles' mainloops (K = 1280 leaves
    enough K rounds for it); integer inputs make the result bit-exact."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", "16")
    Mc, N, K = (2 * tm, 2 * tm, 1280) if P <= 4 else (tm, tm, 1280)
    say(f"gemm_rs band in mainloop P={P} Mc={Mc} N={N} K={K} tile={tm} slot={sdt} grid<=16")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run, slots, out = _gemm_rs(P, Mc, N, K, BF16, sdt, BF16, tm, tm, seed=40 + P + sdt, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.out, BF16), out)
    np.testing.assert_array_equal(bf.to_host(run.win_data, sdt), slots)
    assert torch.all(run.win_flags == run.epoch)


def test_gemm_rs_band_in_mainloop_values(monkeypatch):
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", "24")
    P, Mc, N, K = 8, 256, 512, 1536
    say(f"gemm_rs band in mainloop N(0,1) P={P} Mc={Mc} N={N} K={K} grid<=24")
    run, slots, out = _gemm_rs(P, Mc, N, K, BF16, F32, BF16, 256, 256, seed=77)
    assert relerr(val(bf.to_host(run.out, BF16), BF16), val(out, BF16)) <= TOL[BF16]
    assert relerr(bf.to_host(run.win_data, F32), slots) <= TOL[BF16]


@pytest.mark.parametrize("grid", [1, 5, 13])
def test_gemm_rs_small_grids_integer_bit_exact(grid, monkeypatch):
    """Grids below the queue count (and not a multiple of it): queues without
    a home workgroup are drained by stealing, every band still gets folded."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", str(grid))
    P, Mc, N, K = 4, 512, 512, 256
    say(f"gemm_rs grid={grid} P={P} Mc={Mc} N={N} K={K}")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run, slots, out = _gemm_rs(P, Mc, N, K, BF16, F32, BF16, 256, 256, seed=50 + grid, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.out, BF16), out)
    np.testing.assert_array_equal(bf.to_host(run.win_data, F32), slots)


def _reversed_fold_differs(slots_f32_by_p, out_f32):
    """The inputs are discriminative: folding the same partials in reverse
    rank order gives a different fp32 result somewhere."""
    acc = slots_f32_by_p[-1].astype(np.float32)
    for q in range(len(slots_f32_by_p) - 2, -1, -1):
        acc = (acc + slots_f32_by_p[q].astype(np.float32)).astype(np.float32)
    return bool(np.any(acc != out_f32))


@pytest.mark.parametrize("odt", [F32, BF16])
def test_gemm_rs_reducer_isolation_bit_exact(odt, monkeypatch):
    """Reducer isolation: A_p selects one row of W_p per output row, so every
    partial is an exact bf16 value spread over 2^-20 .. 2^21; the fold is
    then the only rounding, and the GPU's rank-order fp32 fold must equal the
    oracle's bit for bit (a reversed order would not).  A small grid puts
    most folds inside the mainloop."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", "16")
    P, Mc, N, K = 8, 256, 512, 1280
    say(f"gemm_rs reducer isolation P={P} Mc={Mc} N={N} K={K} out={odt}")
    dist = dict(dist_a=("selector",), dist_w=("wide", -20, 20))
    run, slots, out = _gemm_rs(P, Mc, N, K, BF16, F32, odt, 256, 256, seed=90 + odt, dist=dist)
    np.testing.assert_array_equal(bf.to_host(run.win_data, F32), slots)
    np.testing.assert_array_equal(bf.to_host(run.out, odt), out)
    if odt == F32:
        # slots [r][p][Mc][N]: fold destination 0's P partials the other way round
        assert _reversed_fold_differs([slots[0][q] for q in range(P)], out[:Mc])


@pytest.mark.parametrize("P,tm", [(16, 256), (12, 128), (9, 256)])
def test_gemm_rs_many_shards_integer_bit_exact(P, tm):
    """More than 8 shards (up to the ABI's 16): the reducer's wide-P path."""
    Mc, N, K = tm, 2 * tm, 256
    say(f"gemm_rs many shards P={P} Mc={Mc} N={N} K={K} tile={tm}")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run, slots, out = _gemm_rs(P, Mc, N, K, BF16, F32, BF16, tm, tm, seed=100 + P, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.out, BF16), out)
    np.testing.assert_array_equal(bf.to_host(run.win_data, F32), slots)


@pytest.mark.parametrize("sdt", [F32, BF16])
def test_gemm_rs_full_mlpdown_every_element(sdt):
    """The headline workload in the bench's launch configuration, every output
    element and every published slot element against the full oracle."""
    c = cfgs.GEMM_RS_MLP
    say(f"gemm_rs full {c.name} slot={sdt} (every element)")
    A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, BF16, seed=0)
    run = bf.GemmRS(c.P, c.M, c.N, c.K, BF16, sdt, c.out_dt, c.tile_m, c.tile_n, A, W)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    assert torch.all(run.win_flags == run.epoch)
    slots, out = oracle.gemm_rs(c.P, c.M, c.N, c.K, BF16, sdt, c.out_dt, A, W)
    assert relerr(val(bf.to_host(run.out, BF16), BF16), val(out, BF16)) <= TOL[BF16]
    del out
    assert relerr(val(bf.to_host(run.win_data, sdt), sdt), val(slots, sdt)) <= TOL[BF16]


@pytest.mark.parametrize("sdt", [F32, BF16])
def test_gemm_rs_full_mlpdown(sdt):
    c = cfgs.GEMM_RS_MLP
    say(f"gemm_rs full {c.name} slot={sdt} (sampled)")
    A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, BF16, seed=0)
    run = bf.GemmRS(c.P, c.M, c.N, c.K, BF16, sdt, c.out_dt, c.tile_m, c.tile_n, A, W)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    assert torch.all(run.win_flags == run.epoch)
    assert not torch.isnan(run.out.view(torch.bfloat16)).any()
    rng = np.random.default_rng(123)
    n = 3000
    ms = rng.integers(0, c.M, n)
    ns = rng.integers(0, c.N, n)
    # always include tile corners
    ms[:4] = [0, c.M - 1, 1023, 1024]
    ns[:4] = [0, c.N - 1, 255, 256]
    sv, ov = oracle.gemm_rs_points(c.P, c.M, c.N, c.K, BF16, sdt, c.out_dt, A, W, ms, ns)
    out = bf.to_host(run.out, BF16)
    assert relerr(val(out[ms, ns], BF16), val(ov, BF16)) <= TOL[BF16]
    Mc = c.M // c.P
    win = bf.to_host(run.win_data, sdt)       # [r][p][i][n]
    gs = win[ms // Mc, :, ms % Mc, ns]        # [n][P]
    assert relerr(val(gs, sdt), val(sv, sdt)) <= TOL[BF16]


# ====================================================================== GEMM + RS, unfused baseline

UNFUSED_CASES = [
    (4, 64, 256, 256, F32, F32, F32, 64, 64),        # the tiny workload's shapes, fp32
    (4, 300, 328, 136, BF16, F32, BF16, 256, 256),   # ragged, register-staged mainloop
    (3, 300, 328, 136, BF16, BF16, F32, 128, 128),
    (4, 512, 768, 512, BF16, F32, BF16, 256, 256),   # full tiles, direct-to-LDS mainloop
    (8, 256, 512, 1280, BF16, BF16, BF16, 256, 256),
]


@pytest.mark.parametrize("P,Mc,N,K,ind,sdt,odt,tm,tn", UNFUSED_CASES)
def test_gemm_rs_unfused_matches_oracle_and_fused(P, Mc, N, K, ind, sdt, odt, tm, tn):
    """The two-kernel baseline (GEMM, then the fold) gives the oracle's result
    within tolerance and the fused operator's bits exactly: the same tile
    products and the same rank-order fold, only the timing differs.  It
    writes no flags."""
    say(f"gemm_rs unfused P={P} Mc={Mc} N={N} K={K} dt={ind}{sdt}{odt} tile={tm}x{tn}")
    M = P * Mc
    dist = dict(dist_a=("normal", 1.0), dist_w=("normal", 0.02)) if ind == BF16 else \
        dict(dist_a=("uniform",), dist_w=("uniform",))
    A, W = gen.gemm_rs_inputs(P, M, N, K, ind, seed=11 * P + K, **dist)
    u = bf.GemmRS(P, M, N, K, ind, sdt, odt, tm, tn, A, W, unfused=True)
    f = bf.GemmRS(P, M, N, K, ind, sdt, odt, tm, tn, u.A, u.W)
    u.poison()
    f.poison()
    u.run()
    f.run()
    sync()
    assert u.status_value() == 0 and f.status_value() == 0
    slots, out = oracle.gemm_rs(P, M, N, K, ind, sdt, odt, A, W)
    assert relerr(val(bf.to_host(u.out, odt), odt), val(out, odt)) <= TOL[ind]
    assert relerr(val(bf.to_host(u.win_data, sdt), sdt), val(slots, sdt)) <= TOL[ind]
    assert torch.equal(u.out, f.out)
    assert torch.equal(u.win_data, f.win_data)
    assert torch.all(u.win_flags == 0), "the unfused baseline writes no flags"
    assert torch.all(u.ws == 0)


def test_gemm_rs_unfused_integer_bit_exact():
    P, Mc, N, K = 4, 300, 328, 392
    say(f"gemm_rs unfused integer P={P} Mc={Mc} N={N} K={K}")
    M = P * Mc
    A, W = gen.gemm_rs_inputs(P, M, N, K, BF16, seed=12, dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    u = bf.GemmRS(P, M, N, K, BF16, F32, BF16, 256, 256, A, W, unfused=True)
    u.poison()
    u.run()
    sync()
    assert u.status_value() == 0
    slots, out = oracle.gemm_rs(P, M, N, K, BF16, F32, BF16, A, W)
    np.testing.assert_array_equal(bf.to_host(u.out, BF16), out)
    np.testing.assert_array_equal(bf.to_host(u.win_data, F32), slots)


def test_gemm_rs_unfused_full_mlpdown():
    """At the MLP-down workload: bit-identical to the fused operator, and
    sampled outputs against the oracle."""
    c = cfgs.GEMM_RS_MLP
    say(f"gemm_rs unfused full {c.name}")
    A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, BF16, seed=0)
    u = bf.GemmRS(c.P, c.M, c.N, c.K, BF16, F32, c.out_dt, c.tile_m, c.tile_n, A, W, unfused=True)
    u.poison()
    u.run()
    sync()
    assert u.status_value() == 0
    out_u = u.out.clone()
    f = bf.GemmRS(c.P, c.M, c.N, c.K, BF16, F32, c.out_dt, c.tile_m, c.tile_n, u.A, u.W)
    del u
    f.poison()
    f.run()
    sync()
    assert f.status_value() == 0
    assert torch.equal(out_u, f.out)
    rng = np.random.default_rng(7)
    ms = rng.integers(0, c.M, 2000)
    ns = rng.integers(0, c.N, 2000)
    _, ov = oracle.gemm_rs_points(c.P, c.M, c.N, c.K, BF16, F32, c.out_dt, A, W, ms, ns)
    assert relerr(val(bf.to_host(out_u, BF16)[ms, ns], BF16), val(ov, BF16)) <= TOL[BF16]


# ====================================================================== GEMM + AR

def _gemm_ar(P, Mc, N, K, in_dt, slot_dt, out_dt, tm, tn, seed=0, dist=None):
    M = P * Mc
    if dist is None:
        dist = dict(dist_a=("normal", 1.0), dist_w=("normal", 0.02)) if in_dt == BF16 else \
            dict(dist_a=("uniform",), dist_w=("uniform",))
    A, W = gen.gemm_rs_inputs(P, M, N, K, in_dt, seed=seed, **dist)
    run = bf.GemmAR(P, M, N, K, in_dt, slot_dt, out_dt, tm, tn, A, W)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    slots, win = oracle.gemm_ar(P, M, N, K, in_dt, slot_dt, out_dt, A, W)
    return run, slots, win


def _replicas_identical(run):
    """AllReduce: every destination's window holds the same bits."""
    for q in range(1, run.P):
        assert torch.equal(run.out_all[q], run.out_all[0]), f"window {q} differs from window 0"


GEMM_AR_CASES = [
    (4, 64, 256, 256, F32, F32, F32, 64, 64),        # the tiny workload's shapes, fp32
    (3, 100, 200, 76, F32, F32, F32, 64, 64),
    (4, 300, 328, 136, BF16, F32, BF16, 256, 256),
    (3, 300, 328, 136, BF16, BF16, F32, 128, 128),
    (2, 513, 1032, 72, BF16, F32, BF16, 256, 256),
]


@pytest.mark.parametrize("P,Mc,N,K,ind,sdt,odt,tm,tn", GEMM_AR_CASES)
def test_gemm_ar_values(P, Mc, N, K, ind, sdt, odt, tm, tn):
    say(f"gemm_ar P={P} Mc={Mc} N={N} K={K} dt={ind}{sdt}{odt} tile={tm}x{tn}")
    run, slots, win = _gemm_ar(P, Mc, N, K, ind, sdt, odt, tm, tn, seed=3 * P + K)
    assert relerr(val(bf.to_host(run.out_all, odt), odt), val(win, odt)) <= TOL[ind]
    assert relerr(val(bf.to_host(run.win_data, sdt), sdt), val(slots, sdt)) <= TOL[ind]
    _replicas_identical(run)
    assert torch.all(run.win_flags == run.epoch)
    assert torch.all(run.ws == 0)


@pytest.mark.parametrize("P,Mc,N,K,tm,sdt,grid", [
    (4, 300, 328, 392, 256, F32, 0),        # ragged tiles, register-staged mainloop
    (4, 512, 512, 1280, 256, F32, 16),      # bands folded inside later tiles' mainloops
    (8, 256, 256, 1280, 256, BF16, 16),
    (3, 256, 256, 1280, 128, F32, 16),
    (4, 512, 512, 256, 256, F32, 5),        # a grid below the queue count: stealing
    (16, 256, 512, 256, 256, F32, 0),       # the ABI's largest shard count
])
def test_gemm_ar_integer_bit_exact(P, Mc, N, K, tm, sdt, grid, monkeypatch):
    """Integer-valued operands: every partial and fold is exact, so all P
    windows equal the oracle bit for bit, whichever path folds the band."""
    if grid:
        monkeypatch.setenv("HOCF_MAX_WORKGROUPS", str(grid))
    say(f"gemm_ar integer P={P} Mc={Mc} N={N} K={K} tile={tm} slot={sdt} grid={grid or 'full'}")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run, slots, win = _gemm_ar(P, Mc, N, K, BF16, sdt, BF16, tm, tm, seed=200 + P + grid, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.out_all, BF16), win)
    np.testing.assert_array_equal(bf.to_host(run.win_data, sdt), slots)


def test_gemm_ar_reducer_isolation_bit_exact(monkeypatch):
    """Selector operands make every partial an exact bf16 value over 2^-20 ..
    2^21, so the rank-order fp32 fold is the only rounding: all P windows
    must equal the oracle's fold bit for bit (a reversed order would not)."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", "16")
    P, Mc, N, K = 8, 256, 512, 1280
    say(f"gemm_ar reducer isolation P={P} Mc={Mc} N={N} K={K}")
    dist = dict(dist_a=("selector",), dist_w=("wide", -20, 20))
    run, slots, win = _gemm_ar(P, Mc, N, K, BF16, F32, F32, 256, 256, seed=95, dist=dist)
    np.testing.assert_array_equal(bf.to_host(run.win_data, F32), slots)
    np.testing.assert_array_equal(bf.to_host(run.out_all, F32), win)
    assert _reversed_fold_differs([slots[0][q] for q in range(P)], win[0][:Mc])


def test_gemm_ar_full_mlpdown():
    """GEMM + AllReduce at the row-parallel MLP-down shape (P=8, 8192x4096x1792):
    sampled windows against the oracle's fold at those points, all P windows
    bit-identical, every flag set."""
    c = cfgs.GEMM_RS_MLP
    say(f"gemm_ar full {c.name} (sampled)")
    A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, BF16, seed=0)
    run = bf.GemmAR(c.P, c.M, c.N, c.K, BF16, F32, c.out_dt, c.tile_m, c.tile_n, A, W)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    assert torch.all(run.win_flags == run.epoch)
    _replicas_identical(run)
    assert not torch.isnan(run.out_all[0].view(torch.bfloat16)).any()
    rng = np.random.default_rng(321)
    n = 3000
    ms = rng.integers(0, c.M, n)
    ns = rng.integers(0, c.N, n)
    ms[:4] = [0, c.M - 1, 1023, 1024]
    ns[:4] = [0, c.N - 1, 255, 256]
    # the AllReduce's value at (m, n) is the rank-order fold of the P partials there
    _, ov = oracle.gemm_rs_points(c.P, c.M, c.N, c.K, BF16, F32, c.out_dt, A, W, ms, ns)
    out = bf.to_host(run.out_all[c.P - 1], BF16)
    assert relerr(val(out[ms, ns], BF16), val(ov, BF16)) <= TOL[BF16]


# ====================================================================== GEMV + AR

def _gemv(P, Mb, N, K, sdt, odt, tn, seed=0, dist=None):
    dist = dist or {}
    x, W = gen.gemv_ar_inputs(P, Mb, N, K, seed=seed, **dist)
    run = bf.GemvAR(P, Mb, N, K, BF16, sdt, odt, tn, x, W)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    part, win = oracle.gemv_ar(P, Mb, N, K, BF16, sdt, odt, x, W)
    return run, part, win


def test_gemv_ar_decode_config():
    c = cfgs.GEMV_AR_DECODE
    say(f"gemv_ar {c.name}")
    run, part, win = _gemv(c.P, c.Mb, c.N, c.K, c.slot_dt, c.out_dt, c.tile_n)
    got = bf.to_host(run.win_data, c.out_dt)
    for q in range(1, c.P):
        np.testing.assert_array_equal(got[q], got[0])     # replicas bit-identical
    assert relerr(val(got, c.out_dt), val(win, c.out_dt)) <= TOL[BF16]
    assert relerr(val(bf.to_host(run.part, c.slot_dt), c.slot_dt), part) <= TOL[BF16]
    assert torch.all(run.part_flags == run.epoch) and torch.all(run.win_flags == run.epoch)
    assert torch.all(run.ws == 0)


@pytest.mark.parametrize("P,Mb,N,K,sdt,odt,tn", [
    (3, 3, 328, 200, F32, BF16, 128), (5, 1, 1000, 1040, BF16, BF16, 256),
    (2, 8, 1032, 96, F32, F32, 512), (8, 5, 2056, 520, BF16, F32, 256),
])
def test_gemv_ar_ragged(P, Mb, N, K, sdt, odt, tn):
    say(f"gemv_ar ragged P={P} Mb={Mb} N={N} K={K} slot={sdt} out={odt} tile_n={tn}")
    run, part, win = _gemv(P, Mb, N, K, sdt, odt, tn, seed=P * N)
    got = bf.to_host(run.win_data, odt)
    for q in range(1, P):
        np.testing.assert_array_equal(got[q], got[0])
    assert relerr(val(got, odt), val(win, odt)) <= TOL[BF16]


def test_gemv_ar_integer_bit_exact():
    say("gemv_ar integer P=8 Mb=4 N=2048 K=1024")
    ints = dict(dist_x=("int", -2, 2), dist_w=("int", -2, 2))
    run, part, win = _gemv(8, 4, 2048, 1024, F32, BF16, 256, seed=2, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.win_data, BF16), win)
    np.testing.assert_array_equal(bf.to_host(run.part, F32), part)


@pytest.mark.parametrize("grid", [1, 7])
def test_gemv_ar_small_grids_integer_bit_exact(grid, monkeypatch):
    """Each workgroup takes many column tiles in turn (and is the last
    producer of some): still bit-exact, workspace left zeroed."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", str(grid))
    say(f"gemv_ar grid={grid} P=4 Mb=2 N=1024 K=512")
    ints = dict(dist_x=("int", -2, 2), dist_w=("int", -2, 2))
    run, part, win = _gemv(4, 2, 1024, 512, F32, BF16, 128, seed=30 + grid, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.win_data, BF16), win)
    np.testing.assert_array_equal(bf.to_host(run.part, F32), part)
    assert torch.all(run.ws == 0)


def test_gemv_ar_reducer_isolation_bit_exact():
    """x_p selects row b of W_p for output row b: every partial is an exact
    bf16 value of wide magnitude spread, so the rank-order fp32 fold is the
    only rounding and must match the oracle bit for bit."""
    P, Mb, N, K = 8, 4, 2048, 512
    say(f"gemv_ar reducer isolation P={P} Mb={Mb} N={N} K={K}")
    dist = dict(dist_x=("selector",), dist_w=("wide", -20, 20))
    run, part, win = _gemv(P, Mb, N, K, F32, F32, 256, seed=91, dist=dist)
    np.testing.assert_array_equal(bf.to_host(run.part, F32), part)
    np.testing.assert_array_equal(bf.to_host(run.win_data, F32), win)
    assert _reversed_fold_differs([part[q] for q in range(P)], win[0])


@pytest.mark.parametrize("P", [16, 11])
def test_gemv_ar_many_shards_integer_bit_exact(P):
    say(f"gemv_ar many shards P={P} Mb=3 N=1024 K=256")
    ints = dict(dist_x=("int", -2, 2), dist_w=("int", -2, 2))
    run, part, win = _gemv(P, 3, 1024, 256, F32, BF16, 256, seed=110 + P, dist=ints)
    np.testing.assert_array_equal(bf.to_host(run.win_data, BF16), win)
    np.testing.assert_array_equal(bf.to_host(run.part, F32), part)


@pytest.mark.parametrize("P,Mb,N,K,sdt,odt,tn", [
    (8, 4, 8192, 1024, F32, BF16, 256),      # the decode workload
    (3, 3, 328, 200, F32, BF16, 128), (8, 5, 2056, 520, BF16, F32, 256), (16, 2, 1032, 96, F32, F32, 512),
])
def test_gemv_ar_unfused_matches_oracle_and_fused(P, Mb, N, K, sdt, odt, tn):
    """The two-kernel baseline (GEMV, then the fold) gives the oracle's result
    within tolerance and the fused operator's bits exactly, in every window;
    it writes no flags."""
    say(f"gemv_ar unfused P={P} Mb={Mb} N={N} K={K} slot={sdt} out={odt} tile_n={tn}")
    x, W = gen.gemv_ar_inputs(P, Mb, N, K, seed=P + Mb)
    u = bf.GemvAR(P, Mb, N, K, BF16, sdt, odt, tn, x, W, unfused=True)
    f = bf.GemvAR(P, Mb, N, K, BF16, sdt, odt, tn, u.x, u.W)
    u.poison()
    f.poison()
    u.run()
    f.run()
    sync()
    assert u.status_value() == 0 and f.status_value() == 0
    part, win = oracle.gemv_ar(P, Mb, N, K, BF16, sdt, odt, x, W)
    assert relerr(val(bf.to_host(u.win_data, odt), odt), val(win, odt)) <= TOL[BF16]
    assert relerr(val(bf.to_host(u.part, sdt), sdt), val(part, sdt)) <= TOL[BF16]
    assert torch.equal(u.win_data, f.win_data) and torch.equal(u.part, f.part)
    assert torch.all(u.part_flags == 0) and torch.all(u.win_flags == 0)


def test_gemv_ar_unfused_integer_bit_exact():
    P, Mb, N, K = 8, 4, 2048, 1024
    say(f"gemv_ar unfused integer P={P} Mb={Mb} N={N} K={K}")
    x, W = gen.gemv_ar_inputs(P, Mb, N, K, seed=5, dist_x=("int", -2, 2), dist_w=("int", -2, 2))
    u = bf.GemvAR(P, Mb, N, K, BF16, F32, F32, 256, x, W, unfused=True)
    u.poison()
    u.run()
    sync()
    assert u.status_value() == 0
    part, win = oracle.gemv_ar(P, Mb, N, K, BF16, F32, F32, x, W)
    np.testing.assert_array_equal(bf.to_host(u.win_data, F32), win)
    np.testing.assert_array_equal(bf.to_host(u.part, F32), part)


# ====================================================================== GEMM + A2A

def _moe_case(P, E, B, topk, N, K, seed, dist_x=("normal", 1.0), dist_w=("normal", 0.02), tile_m=256):
    off, dest, slot, counts = gen.moe_routing(P, E, B, topk, tile_m, seed=seed)
    X, W = gen.gemm_a2a_inputs(E, int(off[-1]), N, K, dest, seed=seed, dist_x=dist_x, dist_w=dist_w)
    return off, dest, slot, counts, X, W


def _check_a2a(run, want, counts):
    """Rows [0, send_count) of every window hold the oracle's rows; the rest
    was never written (still NaN); every window's flag carries the epoch."""
    got = bf.to_host(run.win_data, run.out_dt)
    for d in range(run.P):
        c = int(counts[d])
        g = val(got[d, :c], run.out_dt)
        assert not np.isnan(g).any(), f"window {d}: unwritten rows"
        if c:
            assert relerr(g, val(want[d, :c], run.out_dt)) <= TOL[BF16]
        assert np.isnan(val(got[d, c:], run.out_dt)).all(), f"window {d}: rows past its count written"
    assert torch.all(run.win_flags[:, 0] == run.epoch)
    assert torch.all(run.ws == 0)


@pytest.mark.parametrize("P,E,B,topk,N,K,odt", [
    (4, 3, 96, 2, 512, 256, BF16), (8, 4, 256, 2, 768, 384, F32), (2, 1, 200, 1, 256, 128, BF16),
    (16, 2, 64, 4, 512, 256, BF16),
])
def test_gemm_a2a_values(P, E, B, topk, N, K, odt):
    say(f"gemm_a2a P={P} E={E} B={B} top{topk} N={N} K={K} out={odt}")
    off, dest, slot, counts, X, W = _moe_case(P, E, B, topk, N, K, seed=P + E + B)
    cap = int(counts.max()) + 8
    run = bf.GemmA2A(P, E, N, K, odt, X, W, off, dest, slot, counts, cap)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    want = oracle.gemm_a2a(P, E, N, K, BF16, odt, X, W, off, dest, slot, cap)
    _check_a2a(run, want, counts)


@pytest.mark.parametrize("tile_m", [128, 256])
def test_gemm_a2a_tile_rows_integer_bit_exact(tile_m):
    """Both row-tile heights (groups padded to 128 or 256 rows) give the
    oracle's bits on integer-valued operands."""
    P, E, B, topk, N, K = 8, 3, 300, 2, 512, 384
    say(f"gemm_a2a tile_m={tile_m} integer P={P} E={E} B={B}")
    off, dest, slot, counts, X, W = _moe_case(P, E, B, topk, N, K, seed=31 + tile_m, dist_x=("int", -2, 2),
                                              dist_w=("int", -2, 2), tile_m=tile_m)
    cap = int(counts.max())
    run = bf.GemmA2A(P, E, N, K, BF16, X, W, off, dest, slot, counts, cap, tile_m=tile_m)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    want = oracle.gemm_a2a(P, E, N, K, BF16, BF16, X, W, off, dest, slot, cap)
    got = bf.to_host(run.win_data, BF16)
    for d in range(P):
        np.testing.assert_array_equal(got[d, :counts[d]], want[d, :counts[d]])
    assert torch.all(run.win_flags[:, 0] == run.epoch)


def test_gemm_a2a_integer_bit_exact_and_repeatable():
    """Integer-valued operands: every row is exact, so the windows equal the
    oracle bit for bit; a second call (new epoch) gives the same bits and
    sets the flags again."""
    P, E, B, topk, N, K = 8, 4, 512, 2, 512, 512
    say(f"gemm_a2a integer P={P} E={E} B={B} N={N} K={K}")
    off, dest, slot, counts, X, W = _moe_case(P, E, B, topk, N, K, seed=21, dist_x=("int", -2, 2),
                                              dist_w=("int", -2, 2))
    cap = int(counts.max())
    run = bf.GemmA2A(P, E, N, K, F32, X, W, off, dest, slot, counts, cap)
    want = oracle.gemm_a2a(P, E, N, K, BF16, F32, X, W, off, dest, slot, cap)
    for call in range(2):
        run.poison()
        run.run()
        sync()
        assert run.status_value() == 0
        got = bf.to_host(run.win_data, F32)
        for d in range(P):
            np.testing.assert_array_equal(got[d, :counts[d]], want[d, :counts[d]], err_msg=f"call {call}")
        assert torch.all(run.win_flags[:, 0] == run.epoch)


def test_gemm_a2a_empty_destination_and_small_grid(monkeypatch):
    """A destination that receives no rows still gets its flag; a grid of a
    few workgroups takes many tiles each."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", "3")
    P, E, N, K = 3, 2, 512, 256
    say(f"gemm_a2a empty destination P={P} E={E} grid<=3")
    rng = np.random.default_rng(4)
    n0, n1 = 300, 140                                # real rows of expert 0 and 1
    off = np.array([0, 512, 768], dtype=np.int64)      # padded to whole 256-row tiles
    dest = np.full(768, -1, dtype=np.int32)
    slot = np.full(768, -1, dtype=np.int32)
    d_real = rng.integers(0, 2, n0 + n1).astype(np.int32)   # destinations 0 and 1 only
    rows = np.concatenate([np.arange(n0), 512 + np.arange(n1)])
    dest[rows] = d_real
    counts = np.bincount(d_real, minlength=P).astype(np.int64)
    for d in range(P):
        m = rows[d_real == d]
        slot[m] = rng.permutation(int(counts[d])).astype(np.int32)
    X, W = gen.gemm_a2a_inputs(E, 768, N, K, dest, seed=4)
    cap = int(counts.max())
    run = bf.GemmA2A(P, E, N, K, BF16, X, W, off, dest, slot, counts, cap)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0 and counts[2] == 0
    want = oracle.gemm_a2a(P, E, N, K, BF16, BF16, X, W, off, dest, slot, cap)
    _check_a2a(run, want, counts)


def test_gemm_a2a_bad_slot_reported_and_skipped():
    P, E, B, topk, N, K = 4, 2, 128, 2, 256, 256
    say(f"gemm_a2a bad slot P={P} E={E} B={B}")
    off, dest, slot, counts, X, W = _moe_case(P, E, B, topk, N, K, seed=8)
    cap = int(counts.max())
    real = np.nonzero(dest >= 0)[0]
    bad = slot.copy()
    victim = int(real[5])
    bad[victim] = cap + 3                       # outside the window: skipped and reported
    run = bf.GemmA2A(P, E, N, K, BF16, X, W, off, dest, bad, counts, cap)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == hocf.HOCF_ERR_BAD_INDEX
    want = oracle.gemm_a2a(P, E, N, K, BF16, BF16, X, W, off, dest, slot, cap)
    got = bf.to_host(run.win_data, BF16)
    d_v, s_v = int(dest[victim]), int(slot[victim])
    ok = np.ones(cap, dtype=bool)
    ok[s_v] = False
    assert np.isnan(val(got[d_v, s_v], BF16)).all()           # the skipped row was not written
    for d in range(P):
        rows_ok = np.arange(int(counts[d])) if d != d_v else np.nonzero(ok[:counts[d]])[0]
        assert relerr(val(got[d, rows_ok], BF16), val(want[d, rows_ok], BF16)) <= TOL[BF16]
    assert int(run.win_flags[d_v, 0]) != run.epoch                # its destination is incomplete
    # the call still leaves the workspace zeroed (the incomplete destination's
    # arrival counter included), so a valid call on it counts from zero
    assert torch.all(run.ws == 0)
    good = bf.GemmA2A(P, E, N, K, BF16, run.X, run.W, off, dest, slot, counts, cap)
    good.ws, good.ws_bytes = run.ws, run.ws_bytes
    good.win_data, good.win_flags, good.win = run.win_data, run.win_flags, run.win
    good.epoch = run.epoch
    run.status.zero_()
    good.status = run.status
    good.poison()
    good.run()
    sync()
    assert good.status_value() == 0
    assert torch.all(good.win_flags[:, 0] == good.epoch)
    _check_a2a(good, want, counts)
    assert torch.all(good.ws == 0)


def test_gemm_a2a_expert_without_rows_and_no_rows_at_all():
    """An expert that received no token (an empty group) is skipped; a call
    with no rows at all still sets every destination's flag and writes
    nothing."""
    P, E, N, K = 4, 3, 256, 256
    say("gemm_a2a empty expert group, then T = 0")
    off, dest, slot, counts = gen.moe_routing(P, 2, 64, 2, 128, seed=6)   # experts 0, 1 ...
    off = np.concatenate([off[:2], off[1:2], off[2:]])                      # ... and an empty expert 1
    X, W = gen.gemm_a2a_inputs(E, int(off[-1]), N, K, dest, seed=6)
    # routing generated for 2 experts: expert 1's rows now belong to expert 2 (its W differs)
    cap = int(counts.max())
    run = bf.GemmA2A(P, E, N, K, BF16, X, W, off, dest, slot, counts, cap, tile_m=128)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    want = oracle.gemm_a2a(P, E, N, K, BF16, BF16, X, W, off, dest, slot, cap)
    _check_a2a(run, want, counts)

    empty = bf.GemmA2A(P, E, N, K, BF16, X[:0], W, np.zeros(E + 1, np.int64), dest[:0], slot[:0],
                       np.zeros(P, np.int64), cap, tile_m=128)
    empty.poison()
    empty.run()
    sync()
    assert empty.status_value() == 0
    assert torch.all(empty.win_flags[:, 0] == empty.epoch)
    assert torch.isnan(empty.win_data.view(torch.bfloat16).float()).all()


def test_gemm_ar_single_shard_and_empty():
    """P = 1: the AllReduce of one partial is the GEMM itself (one window);
    M = 0: nothing is launched, the call succeeds."""
    say("gemm_ar P=1 and M=0")
    ints = dict(dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run, slots, win = _gemm_ar(1, 512, 512, 256, BF16, F32, F32, 256, 256, seed=3, dist=ints)
    A = bf.to_host(run.A, BF16)
    Wm = bf.to_host(run.W, BF16)
    plain = (val(A[0], BF16) @ val(Wm[0], BF16)).astype(np.float32)
    np.testing.assert_array_equal(bf.to_host(run.out_all, F32)[0], plain)
    e = bf.GemmAR(2, 0, 256, 256, BF16, F32, BF16, 256, 256, A[:, :0].repeat(2, 0)[:2], Wm.repeat(2, 0))
    assert e.call() == hocf.HOCF_OK


def test_gemm_a2a_most_experts_and_destinations():
    """The ABI's limits: 64 local experts (64 groups of one mostly padded
    tile each) and 16 destination ranks; integer operands, bit-exact."""
    P, E, B, topk, N, K = 16, 64, 96, 4, 256, 128
    say(f"gemm_a2a limits P={P} E={E} B={B} top{topk}")
    off, dest, slot, counts, X, W = _moe_case(P, E, B, topk, N, K, seed=64, dist_x=("int", -2, 2),
                                              dist_w=("int", -2, 2))
    cap = int(counts.max())
    run = bf.GemmA2A(P, E, N, K, F32, X, W, off, dest, slot, counts, cap)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    want = oracle.gemm_a2a(P, E, N, K, BF16, F32, X, W, off, dest, slot, cap)
    got = bf.to_host(run.win_data, F32)
    for d in range(P):
        np.testing.assert_array_equal(got[d, :counts[d]], want[d, :counts[d]])
    assert torch.all(run.win_flags[:, 0] == run.epoch)


@pytest.mark.parametrize("grid,parts", [(8, 2), (16, 4), (32, 2)])
def test_gemm_a2a_last_round_in_part_tiles_bit_exact(grid, parts, monkeypatch):
    """A grid that leaves a partial last round: those tiles run as quarter-
    height tiles when four times their number fits one round of the grid,
    else as half-height tiles (every row still computed once); integer
    operands, bit-exact, every flag set."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", str(grid))
    P, E, B, topk, N, K = 8, 3, 400, 2, 1024, 256
    off, dest, slot, counts, X, W = _moe_case(P, E, B, topk, N, K, seed=70 + grid, dist_x=("int", -2, 2),
                                              dist_w=("int", -2, 2))
    tiles = int(off[-1]) // 256 * (N // 256)
    rem = tiles % grid
    say(f"gemm_a2a part tiles: {tiles} tiles on a grid of {grid} (remainder {rem}, {parts} parts)")
    assert 0 < rem and (4 * rem <= grid if parts == 4 else grid < 4 * rem <= 2 * grid)
    cap = int(counts.max())
    run = bf.GemmA2A(P, E, N, K, BF16, X, W, off, dest, slot, counts, cap)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    want = oracle.gemm_a2a(P, E, N, K, BF16, BF16, X, W, off, dest, slot, cap)
    got = bf.to_host(run.win_data, BF16)
    for d in range(P):
        np.testing.assert_array_equal(got[d, :counts[d]], want[d, :counts[d]])
    assert torch.all(run.win_flags[:, 0] == run.epoch)


def test_gemm_a2a_full_moe():
    """The MoE combine workload: 8 ranks x 4096 tokens, top-2 of 32 experts,
    this rank's 4 experts (K=1792 -> N=4096): every window row against the
    oracle."""
    c = cfgs.GEMM_A2A_MOE
    say(f"gemm_a2a full {c.name} tile {c.tile_m}x{c.tile_n}")
    off, dest, slot, counts, X, W = _moe_case(c.P, c.E, c.B, c.topk, c.N, c.K, seed=0, tile_m=c.tile_m)
    run = bf.GemmA2A(c.P, c.E, c.N, c.K, BF16, X, W, off, dest, slot, counts, c.cap, tile_m=c.tile_m)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    want = oracle.gemm_a2a(c.P, c.E, c.N, c.K, BF16, BF16, X, W, off, dest, slot, c.cap)
    _check_a2a(run, want, counts)


# ====================================================================== AG + GEMM

def _ag_inputs(P, Mc, N, K, seed=0):
    return gen.ag_gemm_inputs(P, Mc, N, K, seed=seed)


@pytest.mark.parametrize("P,Mc,N,K,tm,odt", [(3, 300, 328, 136, 128, BF16), (4, 300, 520, 200, 256, F32),
                                             (8, 128, 256, 64, 128, BF16)])
def test_ag_gemm_release_orders(P, Mc, N, K, tm, odt):
    """Chunk flags set by the host (coherent pinned memory) while the kernel runs,
    in three different orders, plus flags pre-released on the kernel's stream:
    every output must be bit-identical and match the oracle."""
    say(f"ag_gemm P={P} Mc={Mc} N={N} K={K} tile={tm} out={odt}: 3 host release orders + pre-release")
    chunks, W, order = _ag_inputs(P, Mc, N, K, seed=P + N)
    run = bf.AgGemm(P, Mc, N, K, odt, tm, tm, chunks, W, flags="host")
    outs = []
    for o in (order, np.arange(P), np.arange(P)[::-1]):
        run.poison()
        run.run_host_released(o, delay_s=0.0005)
        sync()
        assert run.status_value() == 0
        outs.append(run.out.clone())
    pre = bf.AgGemm(P, Mc, N, K, odt, tm, tm, run.A, run.W, flags="device")
    pre.poison()
    pre.run_prereleased(order)
    sync()
    assert pre.status_value() == 0
    outs.append(pre.out.clone())
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "output depends on the release order"
    _, want = oracle.ag_gemm(P, Mc, N, K, BF16, odt, list(chunks), W)
    assert relerr(val(bf.to_host(outs[0], odt), odt), val(want, odt)) <= TOL[BF16]
    assert torch.all(run.ws == 0) and torch.all(pre.ws == 0)


def test_ag_gemm_integer_bit_exact():
    say("ag_gemm integer P=4 Mc=256 N=512 K=512")
    P, Mc, N, K = 4, 256, 512, 512
    chunks, W, order = gen.ag_gemm_inputs(P, Mc, N, K, seed=5, dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run = bf.AgGemm(P, Mc, N, K, BF16, 256, 256, chunks, W)
    run.poison()
    run.run_prereleased(order)
    sync()
    _, want = oracle.ag_gemm(P, Mc, N, K, BF16, BF16, list(chunks), W)
    np.testing.assert_array_equal(bf.to_host(run.out, BF16), want)


@pytest.mark.parametrize("grid", [1, 3])
def test_ag_gemm_small_grids_integer_bit_exact(grid, monkeypatch):
    """Fewer workgroups than tiles: every workgroup draws tickets after its
    first (the counter's range), chunks are registered once; bit-exact."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", str(grid))
    P, Mc, N, K = 4, 256, 512, 512
    say(f"ag_gemm grid={grid} P={P} Mc={Mc} N={N} K={K}")
    chunks, W, order = gen.ag_gemm_inputs(P, Mc, N, K, seed=60 + grid, dist_a=("int", -2, 2),
                                          dist_w=("int", -2, 2))
    run = bf.AgGemm(P, Mc, N, K, BF16, 256, 256, chunks, W)
    run.poison()
    run.run_prereleased(order)
    sync()
    assert run.status_value() == 0
    _, want = oracle.ag_gemm(P, Mc, N, K, BF16, BF16, list(chunks), W)
    np.testing.assert_array_equal(bf.to_host(run.out, BF16), want)
    assert torch.all(run.ws == 0)


def test_ag_gemm_sixteen_chunks_integer_bit_exact():
    P, Mc, N, K = 16, 128, 256, 256
    say(f"ag_gemm P={P} Mc={Mc} N={N} K={K}")
    chunks, W, order = gen.ag_gemm_inputs(P, Mc, N, K, seed=120, dist_a=("int", -2, 2), dist_w=("int", -2, 2))
    run = bf.AgGemm(P, Mc, N, K, BF16, 128, 128, chunks, W)
    run.poison()
    run.run_prereleased(order)
    sync()
    assert run.status_value() == 0
    _, want = oracle.ag_gemm(P, Mc, N, K, BF16, BF16, list(chunks), W)
    np.testing.assert_array_equal(bf.to_host(run.out, BF16), want)
    assert torch.all(run.ws == 0)


def test_ag_gemm_late_delivery():
    """The chunks live in coherent pinned host memory and start as NaN; after the
    kernel has started, the host writes chunk c's data and then its flag, one
    chunk every 2 ms.  Any read of a chunk before its flag shows up as NaN."""
    P, Mc, N, K = 4, 256, 384, 256
    say(f"ag_gemm late delivery from the host P={P} Mc={Mc} N={N} K={K}")
    chunks, W, order = _ag_inputs(P, Mc, N, K, seed=11)
    run = bf.AgGemm(P, Mc, N, K, BF16, 128, 128, None, W, flags="host", chunks_on_host=True)
    run.host_chunks[:] = 0x7FC0
    run.poison()

    def deliver(c):
        run.host_chunks[c] = chunks[c]

    run.run_host_released(order, delay_s=0.002, deliver=deliver, spin_timeout_ns=2_000_000_000)
    sync()
    assert run.status_value() == 0
    _, want = oracle.ag_gemm(P, Mc, N, K, BF16, BF16, list(chunks), W)
    assert relerr(val(bf.to_host(run.out, BF16), BF16), val(want, BF16)) <= TOL[BF16]


def test_ag_gemm_withheld_chunk_times_out():
    """A chunk whose flag never arrives: the waiting workgroups give up after the
    (tiny) time limit, record HOCF_ERR_TIMEOUT and exit; the other chunks' tiles
    are still right, and the next call with all chunks succeeds."""
    P, Mc, N, K = 4, 256, 256, 128
    say(f"ag_gemm withheld chunk (timeout 20 ms) P={P}")
    chunks, W, _ = _ag_inputs(P, Mc, N, K, seed=4)
    run = bf.AgGemm(P, Mc, N, K, BF16, 128, 128, chunks, W, flags="host")
    run.poison()
    run.run_host_released([0, 2, 3], spin_timeout_ns=20_000_000)
    sync()
    assert run.status_value() == hocf.HOCF_ERR_TIMEOUT
    _, want = oracle.ag_gemm(P, Mc, N, K, BF16, BF16, list(chunks), W)
    got = val(bf.to_host(run.out, BF16), BF16)
    for c in (0, 2, 3):
        rows = slice(c * Mc, (c + 1) * Mc)
        assert relerr(got[rows], val(want, BF16)[rows]) <= TOL[BF16]
    assert torch.all(run.ws == 0), "a timed-out call must still leave the workspace zeroed"
    run.status.zero_()
    run.poison()
    run.run_host_released([3, 1, 0, 2])
    sync()
    assert run.status_value() == 0
    assert relerr(val(bf.to_host(run.out, BF16), BF16), val(want, BF16)) <= TOL[BF16]


def test_ag_gemm_abort():
    """A withheld chunk and a host-pinned abort word set by the host 10 ms in:
    the waiting workgroups record HOCF_ERR_ABORTED and exit."""
    P, Mc, N, K = 2, 128, 128, 64
    say("ag_gemm abort word set by the host, chunk withheld")
    chunks, W, _ = _ag_inputs(P, Mc, N, K, seed=6)
    run = bf.AgGemm(P, Mc, N, K, BF16, 128, 128, chunks, W, flags="host")
    addr, _ = hocf.host_coherent(4)
    abort = np.frombuffer(bf.ctypes_char_array(addr, 4), dtype=np.uint32)
    run.run_host_released([0], abort_flag=addr, spin_timeout_ns=5_000_000_000)
    import time
    time.sleep(0.01)
    abort[0] = 1
    sync()
    assert run.status_value() == hocf.HOCF_ERR_ABORTED
    assert torch.all(run.ws == 0)


def test_ag_gemm_full_colpar():
    c = cfgs.AG_GEMM_COL
    say(f"ag_gemm full {c.name} (every element; pre-released and host-released orders)")
    chunks, W, order = _ag_inputs(c.P, c.Mc, c.N, c.K, seed=0)
    run = bf.AgGemm(c.P, c.Mc, c.N, c.K, BF16, c.tile_m, c.tile_n, chunks, W)
    run.poison()
    run.run_prereleased(order)
    sync()
    assert run.status_value() == 0
    host = bf.AgGemm(c.P, c.Mc, c.N, c.K, BF16, c.tile_m, c.tile_n, run.A, run.W, flags="host")
    host.poison()
    host.run_host_released(np.arange(c.P)[::-1], delay_s=0.0002)
    sync()
    assert host.status_value() == 0
    assert torch.equal(run.out, host.out)
    _, want = oracle.ag_gemm(c.P, c.Mc, c.N, c.K, BF16, BF16, list(chunks), W)   # every element
    assert relerr(val(bf.to_host(run.out, BF16), BF16), val(want, BF16)) <= TOL[BF16]
    assert not torch.isnan(run.out.view(torch.bfloat16)).any()


# ====================================================================== emb-bag + A2A

def _emb_check(run, T, R, D, B, L, P, tables, idx, off=None):
    win = oracle.embbag_a2a(T, R, D, B, L, P, tables, idx, off)
    got = run.win_data.cpu().numpy()
    np.testing.assert_array_equal(got, win)      # sequential fp32 sums: bit-exact
    assert torch.all(run.win_flags == run.epoch)


@pytest.mark.parametrize("D,tile_bags", [(128, 16), (64, 7), (200, 32), (512, 64), (4, 1)])
def test_embbag_values_bit_exact(D, tile_bags):
    T, R, B, L, P = 5, 3000, 96, 13, 4
    say(f"embbag T={T} R={R} D={D} B={B} L={L} P={P} tile_bags={tile_bags}")
    tables = gen.embbag_tables(T, R, D, std=0.01, seed=D)
    idx = gen.zipf_indices(T, B, L, R, seed=D)
    run = bf.EmbbagA2A(T, R, D, B, L, P, tile_bags, tables, idx)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    _emb_check(run, T, R, D, B, L, P, tables, idx)
    assert torch.all(run.ws == 0)


@pytest.mark.parametrize("grid", [1, 6])
def test_embbag_small_grids_bit_exact(grid, monkeypatch):
    """Each workgroup pools many tiles of bags (and steals from other
    queues): every (bag, table) lands once, bit-exact, workspace zeroed."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", str(grid))
    T, R, D, B, L, P = 4, 2000, 128, 128, 9, 4
    say(f"embbag grid={grid} T={T} R={R} D={D} B={B} L={L} P={P}")
    tables = gen.embbag_tables(T, R, D, std=0.01, seed=70 + grid)
    idx = gen.zipf_indices(T, B, L, R, seed=70 + grid)
    run = bf.EmbbagA2A(T, R, D, B, L, P, 8, tables, idx)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    _emb_check(run, T, R, D, B, L, P, tables, idx)
    assert torch.all(run.ws == 0)


def test_embbag_sixteen_destinations_bit_exact():
    T, R, D, B, L, P = 3, 4000, 128, 256, 11, 16
    say(f"embbag P={P} T={T} R={R} D={D} B={B} L={L}")
    tables = gen.embbag_tables(T, R, D, std=0.01, seed=130)
    idx = gen.zipf_indices(T, B, L, R, seed=130)
    run = bf.EmbbagA2A(T, R, D, B, L, P, 8, tables, idx)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    _emb_check(run, T, R, D, B, L, P, tables, idx)


def test_embbag_tagged_routing():
    T, R, D, B, L, P = 6, 20000, 128, 512, 20, 8
    say("embbag tagged tables: routing, table and index use bit-exact")
    tables = gen.tagged_tables(T, R, D)
    idx = gen.zipf_indices(T, B, L, R, seed=1)
    run = bf.EmbbagA2A(T, R, D, B, L, P, 16, tables, idx)
    run.poison()
    run.run()
    sync()
    _emb_check(run, T, R, D, B, L, P, tables, idx)


def test_embbag_csr_ragged_and_empty():
    T, R, D, B, P = 3, 5000, 128, 200, 4
    say("embbag CSR bags of 0..45 rows (some empty)")
    off = gen.csr_bag_offsets(T, B, 45, seed=2, empty_frac=0.15)
    idx = np.random.default_rng(3).integers(0, R, size=int(off[-1]), dtype=np.int32)
    tables = gen.embbag_tables(T, R, D, std=1.0, seed=4)
    run = bf.EmbbagA2A(T, R, D, B, 0, P, 8, tables, idx, off)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    _emb_check(run, T, R, D, B, 0, P, tables, idx, off)


def test_embbag_bad_index_reported_and_skipped():
    T, R, D, B, L, P = 2, 100, 128, 16, 4, 2
    say("embbag out-of-range index")
    tables = gen.embbag_tables(T, R, D, std=1.0, seed=5)
    idx = gen.uniform_indices(T, B, L, R, seed=6)
    idx[1, 3, 2] = R          # one bad index
    idx[0, 0, 0] = -5         # and a negative one
    run = bf.EmbbagA2A(T, R, D, B, L, P, 4, tables, idx)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == hocf.HOCF_ERR_BAD_INDEX
    # the bags sum their valid rows: same as the oracle on the bags with the bad entries dropped
    off = np.zeros(T * B + 1, np.int64)
    keep = []
    for t in range(T):
        for b in range(B):
            rows = [r for r in idx[t, b] if 0 <= r < R]
            keep += rows
            off[t * B + b + 1] = off[t * B + b] + len(rows)
    want = oracle.embbag_a2a(T, R, D, B, 0, P, tables, np.asarray(keep, np.int32), off)
    np.testing.assert_array_equal(run.win_data.cpu().numpy(), want)


def test_embbag_full_dlrm():
    c = cfgs.EMBBAG_DLRM
    say(f"embbag full {c.name} (tables drawn on the GPU, sampled bags bit-exact)")
    tables = gen.embbag_tables_torch(c.T, c.R, c.D, seed=0)
    idx = gen.zipf_indices(c.T, c.B, c.L, c.R, alpha=c.alpha, seed=0)
    run = bf.EmbbagA2A(c.T, c.R, c.D, c.B, c.L, c.P, c.tile_bags, tables, idx)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    assert torch.all(run.win_flags == run.epoch)
    assert not torch.isnan(run.win_data).any()
    rng = np.random.default_rng(9)
    ts = rng.integers(0, c.T, 2048)
    bs = rng.integers(0, c.B, 2048)
    # the sampled bags' rows, copied back from the device tables, as one small table
    rows = idx[ts, bs]                                        # [n][L]
    flat = torch.from_numpy(rows.reshape(-1).astype(np.int64)).cuda()
    tsel = torch.from_numpy(np.repeat(ts, c.L).astype(np.int64)).cuda()
    mini = tables[tsel, flat].cpu().numpy()[None]             # [1][n*L][D]
    n = len(ts)
    midx = np.arange(n * c.L, dtype=np.int32).reshape(1, n, c.L)
    want = oracle.embbag_a2a(1, n * c.L, c.D, n, c.L, 1, mini, midx)[0, :, 0]   # [n][D]
    Bd = c.B // c.P
    got = run.win_data[torch.from_numpy(bs // Bd).cuda(), torch.from_numpy(bs % Bd).cuda(),
                       torch.from_numpy(ts).cuda()].cpu().numpy()
    np.testing.assert_array_equal(got, want)
    del tables
    torch.cuda.empty_cache()


# ====================================================================== determinism

def _repeat_identical(run_call, outs, n=1000):
    """n calls, each output compared on the device with the first call's: every
    call must give the same bits (fixed reduction order, no arrival dependence)."""
    run_call(0)
    sync()
    refs = [o.clone() for o in outs()]
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for i in range(1, n):
        run_call(i)
        for o, r in zip(outs(), refs):
            bad += (o.view(torch.int32 if o.element_size() == 4 else torch.int16) !=
                    r.view(torch.int32 if r.element_size() == 4 else torch.int16)).any()
    sync()
    return int(bad.item())


@pytest.mark.parametrize("op", ["gemm_rs", "gemm_ar", "gemm_rs_unfused", "gemv_ar", "ag_gemm", "embbag_a2a",
                                "gemm_a2a"])
def test_thousand_calls_bit_identical(op, monkeypatch):
    """1000 calls of each operator on one buffer set give bit-identical results
    (outputs NaN-poisoned before every call).  A small grid makes the GEMM
    reductions fold bands inside later tiles' mainloops, in whichever order
    the workgroups happen to run; AllGather+GEMM cycles through six chunk
    release orders."""
    monkeypatch.setenv("HOCF_MAX_WORKGROUPS", "24")
    say(f"{op}: 1000 calls bit-identical")
    if op in ("gemm_rs", "gemm_ar", "gemm_rs_unfused"):
        P, Mc, N, K = 4, 512, 512, 1280
        A, W = gen.gemm_rs_inputs(P, P * Mc, N, K, BF16, seed=13)
        if op == "gemm_ar":
            r = bf.GemmAR(P, P * Mc, N, K, BF16, F32, BF16, 256, 256, A, W)
            outs = lambda: [r.out_all]
        else:
            r = bf.GemmRS(P, P * Mc, N, K, BF16, F32, BF16, 256, 256, A, W, unfused=op == "gemm_rs_unfused")
            outs = lambda: [r.out]
        call = lambda i: (r.poison(), r.run())
    elif op == "gemv_ar":
        x, W = gen.gemv_ar_inputs(8, 4, 2048, 1024, seed=13)
        r = bf.GemvAR(8, 4, 2048, 1024, BF16, F32, BF16, 256, x, W)
        outs = lambda: [r.win_data]
        call = lambda i: (r.poison(), r.run())
    elif op == "ag_gemm":
        chunks, W, _ = gen.ag_gemm_inputs(4, 256, 512, 512, seed=13)
        r = bf.AgGemm(4, 256, 512, 512, BF16, 256, 256, chunks, W)
        orders = [np.random.default_rng(k).permutation(4) for k in range(6)]
        outs = lambda: [r.out]
        call = lambda i: (r.poison(), r.run_prereleased(orders[i % 6]))
    elif op == "embbag_a2a":
        T, R, D, B, L = 4, 5000, 128, 512, 20
        tab = gen.embbag_tables(T, R, D, seed=13)
        idx = gen.zipf_indices(T, B, L, R, seed=13)
        r = bf.EmbbagA2A(T, R, D, B, L, 8, 16, tab, idx)
        outs = lambda: [r.win_data]
        call = lambda i: (r.poison(), r.run())
    else:
        off, dest, slot, counts, X, W = _moe_case(8, 4, 256, 2, 512, 512, seed=13)
        r = bf.GemmA2A(8, 4, 512, 512, BF16, X, W, off, dest, slot, counts, int(counts.max()))
        outs = lambda: [r.win_data]
        call = lambda i: (r.poison(), r.run())
    assert _repeat_identical(call, outs) == 0
    assert r.status_value() == 0


# ====================================================================== A2A + GEMM (MoE dispatch)

def _a2g_case(P, E, e0, B, topk, N, K, seed, dist=None):
    experts = gen.moe_choices(P, E, B, topk, seed=seed)
    X, W = gen.a2a_gemm_inputs(P, B, K, E, N, seed=seed, **(dist or {}))
    return experts, X, W


def _a2g_check(run, want, integer=False):
    """Layout, received rows and dest/slot bit-exact; Y within tolerance (bit-exact
    for integer inputs); rows past the groups untouched (poison)."""
    recv_o, Y_o, off_o, dest_o, slot_o, cnt_o = want
    off = run.offsets.cpu().numpy()
    np.testing.assert_array_equal(off, off_o)
    np.testing.assert_array_equal(run.send_counts.cpu().numpy(), cnt_o)
    T = int(off[-1])
    np.testing.assert_array_equal(run.dest.cpu().numpy()[:T], dest_o[:T])
    np.testing.assert_array_equal(run.slot.cpu().numpy()[:T], slot_o[:T])
    np.testing.assert_array_equal(bf.to_host(run.recv, BF16)[:T], recv_o[:T])
    Y = bf.to_host(run.Y, run.out_dt)
    if T:
        if integer:
            np.testing.assert_array_equal(Y[:T], Y_o[:T])
        else:
            assert relerr(val(Y[:T], run.out_dt), val(Y_o[:T], run.out_dt)) <= TOL[BF16]
    assert np.all(run.dest.cpu().numpy()[T:] == -77), "rows past the groups were written"
    if T < run.cap:
        assert np.isnan(val(Y[T:], run.out_dt)).all()


@pytest.mark.parametrize("P,E,e0,B,topk,N,K,odt,tm", [
    (2, 2, 0, 100, 2, 256, 128, BF16, 256),      # one row tile per expert, mostly padding
    (4, 3, 3, 300, 2, 512, 256, F32, 256),       # this rank owns experts 3..5 of 12
    (3, 2, 2, 700, 3, 256, 384, BF16, 128),      # 128-row groups; chunks straddle tokens (topk 3)
    (8, 4, 0, 512, 2, 768, 512, BF16, 256),
])
def test_a2a_gemm_values(P, E, e0, B, topk, N, K, odt, tm):
    say(f"a2a_gemm P={P} E={E} e0={e0} B={B} topk={topk} N={N} K={K} out={odt} tile={tm}")
    experts, X, W = _a2g_case(P, E, e0, B, topk, N, K, seed=P + E + B)
    cap = P * B * topk // 2 + E * tm
    run = bf.A2aGemm(P, E, e0, B, topk, N, K, odt, X, experts, W, cap, tile_m=tm)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    want = oracle.a2a_gemm(P, E, e0, B, topk, N, K, BF16, odt, X, experts, W, tm, cap)
    _a2g_check(run, want)


@pytest.mark.parametrize("grid", [0, 1, 3])
def test_a2a_gemm_integer_bit_exact_and_unfused_identical(grid, monkeypatch):
    """Integer inputs: Y bit-exact.  With a grid of one or a few workgroups
    every tile's rows come from items the same few workgroups claimed
    earlier (the kernel needs no co-residency).  The unfused pair (scatter
    kernel, then GEMM kernel) gives the same bits."""
    if grid:
        monkeypatch.setenv("HOCF_MAX_WORKGROUPS", str(grid))
    P, E, e0, B, topk, N, K = 4, 2, 2, 400, 2, 512, 256
    say(f"a2a_gemm integer, grid cap {grid}")
    ints = dict(dist_x=("int", -2, 2), dist_w=("int", -2, 2))
    experts, X, W = _a2g_case(P, E, e0, B, topk, N, K, seed=77, dist=ints)
    cap = 1024
    run = bf.A2aGemm(P, E, e0, B, topk, N, K, F32, X, experts, W, cap)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    want = oracle.a2a_gemm(P, E, e0, B, topk, N, K, BF16, F32, X, experts, W, 256, cap)
    _a2g_check(run, want, integer=True)
    un = bf.A2aGemm(P, E, e0, B, topk, N, K, F32, run.X, run.experts, run.W, cap, unfused=True)
    un.poison()
    un.run()
    sync()
    assert un.status_value() == 0
    T = int(run.offsets[-1])
    assert torch.equal(un.Y[:T], run.Y[:T]) and torch.equal(un.recv[:T], run.recv[:T])
    assert torch.equal(un.dest, run.dest) and torch.equal(un.slot, run.slot)
    assert torch.equal(un.offsets, run.offsets) and torch.equal(un.send_counts, run.send_counts)


def test_a2a_gemm_capacity_and_no_local_pairs():
    """More rows than the receive buffer holds: HOCF_ERR_CAPACITY, no row
    delivered, no tile computed; then the same object with every choice
    elsewhere: empty groups, zero send counts, nothing written."""
    P, E, B, topk, N, K = 4, 2, 256, 2, 256, 128
    say("a2a_gemm capacity exceeded, then no local pairs")
    experts, X, W = _a2g_case(P, E, 0, B, topk, N, K, seed=5)
    run = bf.A2aGemm(P, E, 0, B, topk, N, K, BF16, X, experts, W, cap=256)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == hocf.HOCF_ERR_CAPACITY
    assert torch.all(run.dest == -77)
    assert torch.isnan(run.Y.view(torch.bfloat16).float()).all()
    none = torch.full_like(run.experts, 99)
    empty = bf.A2aGemm(P, E, 0, B, topk, N, K, BF16, run.X, none, run.W, cap=256)
    empty.poison()
    empty.run()
    sync()
    assert empty.status_value() == 0
    assert empty.offsets.cpu().tolist() == [0] * (E + 1)
    assert empty.send_counts.cpu().tolist() == [0] * P
    assert torch.all(empty.dest == -77)


def test_a2a_gemm_full_moe_dispatch_every_element():
    """The MoE dispatch workload (8 ranks x 4096 tokens, top-2 of 32 experts,
    this rank's 4 experts 4096 -> 1792) in the bench's launch configuration:
    layout and received rows bit-exact, every Y element against the oracle,
    and 20 repeated calls bit-identical."""
    c = cfgs.A2A_GEMM_MOE
    say(f"a2a_gemm full {c.name}")
    experts, X, W = _a2g_case(c.P, c.E, 0, c.B, c.topk, c.N, c.K, seed=0)
    run = bf.A2aGemm(c.P, c.E, 0, c.B, c.topk, c.N, c.K, BF16, X, experts, W, c.cap, tile_m=c.tile_m)
    run.poison()
    run.run()
    sync()
    assert run.status_value() == 0
    want = oracle.a2a_gemm(c.P, c.E, 0, c.B, c.topk, c.N, c.K, BF16, BF16, X, experts, W, c.tile_m, c.cap)
    _a2g_check(run, want)
    first = run.Y.clone()
    for _ in range(20):
        run.run()
    sync()
    assert run.status_value() == 0
    assert torch.equal(run.Y, first)


def test_a2a_gemm_alternating_inputs_no_stale_reads():
    """Two different routings and token sets on the same receive and output
    buffers, one call after the other, three times: every call matches its
    own oracle (the tiles never read received rows left by the previous
    call from an XCD's L2)."""
    P, E, B, topk, N, K = 4, 2, 512, 2, 512, 256
    say("a2a_gemm alternating inputs on the same buffers")
    cases = [_a2g_case(P, E, 0, B, topk, N, K, seed=s) for s in (101, 202)]
    wants = [oracle.a2a_gemm(P, E, 0, B, topk, N, K, BF16, BF16, X, ex_, W, 256, 2048) for ex_, X, W in cases]
    run = bf.A2aGemm(P, E, 0, B, topk, N, K, BF16, cases[0][1], cases[0][0], cases[0][2], 2048)
    dev = [(bf.to_device(X), bf.to_device(np.ascontiguousarray(ex_, np.int32)), bf.to_device(W)) for ex_, X, W in cases]
    for k in range(6):
        run.X, run.experts, run.W = dev[k % 2]
        run.dest.fill_(-77)          # (recv is not touched between the calls)
        bf.nan_fill(run.Y)
        run.run()
        sync()
        assert run.status_value() == 0
        _a2g_check(run, wants[k % 2])


# ====================================================================== GEMM + RS, decomposed (InterDecom)

@pytest.mark.parametrize("pieces,fold_cus", [(1, 0), (2, 32), (4, 0), (4, 64), (8, 32)])
def test_gemm_rs_decomposed_identical_to_fused(pieces, fold_cus):
    """Column pieces pipelined on two streams give the fused operator's bits
    (output and every slot): the same tile products, the same fold."""
    P, Mc, N, K = 4, 512, 2048, 512
    say(f"gemm_rs decomposed pieces={pieces} fold_cus={fold_cus}")
    A, W = gen.gemm_rs_inputs(P, P * Mc, N, K, BF16, seed=pieces)
    fused = bf.GemmRS(P, P * Mc, N, K, BF16, F32, BF16, 256, 256, A, W)
    fused.poison()
    fused.run()
    dec = bf.GemmRS(P, P * Mc, N, K, BF16, F32, BF16, 256, 256, fused.A, fused.W, pieces=pieces, fold_cus=fold_cus)
    dec.poison()
    dec.run()
    sync()
    assert fused.status_value() == 0 and dec.status_value() == 0
    assert torch.equal(dec.out, fused.out)
    assert torch.equal(dec.win_data, fused.win_data)
    _, out = oracle.gemm_rs(P, P * Mc, N, K, BF16, F32, BF16, A, W, want_slots=False)
    assert relerr(val(bf.to_host(dec.out, BF16), BF16), val(out, BF16)) <= TOL[BF16]


def test_gemm_rs_decomposed_tiny_fp32_and_full_mlpdown():
    """The tiny fp32 workload in 4 pieces of 64 columns, and the MLP-down
    workload in 4 pieces with 32 CUs left to the folds: bit-identical to
    the fused operator."""
    c = cfgs.GEMM_RS_TINY
    say(f"gemm_rs decomposed {c.name} pieces=4")
    A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, F32, seed=0, dist_a=c.dist_a, dist_w=c.dist_w)
    f = bf.GemmRS(c.P, c.M, c.N, c.K, F32, F32, F32, 64, 64, A, W)
    d = bf.GemmRS(c.P, c.M, c.N, c.K, F32, F32, F32, 64, 64, f.A, f.W, pieces=4, fold_cus=16)
    f.poison(); d.poison()
    f.run(); d.run()
    sync()
    assert torch.equal(d.out, f.out)
    c = cfgs.GEMM_RS_MLP
    say(f"gemm_rs decomposed {c.name} pieces=4 fold_cus=32")
    A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, BF16, seed=0)
    f = bf.GemmRS(c.P, c.M, c.N, c.K, BF16, F32, BF16, 256, 256, A, W)
    d = bf.GemmRS(c.P, c.M, c.N, c.K, BF16, F32, BF16, 256, 256, f.A, f.W, pieces=4, fold_cus=32)
    f.poison(); d.poison()
    f.run(); d.run()
    sync()
    assert f.status_value() == 0 and d.status_value() == 0
    assert torch.equal(d.out, f.out)
