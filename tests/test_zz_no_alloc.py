"""The GEMM + ReduceScatter entry point that allocates nothing
(hocf_gemm_rs_noalloc, the library's per-device scratch in place of a
workspace) against hocf_gemm_rs: the same output and slot bits and the
oracle's values, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's words; each call clears what it uses)."""

import numpy as np
import pytest
import torch

import oracle
from computation_collective_amd import buffers as bf
from computation_collective_amd import hocf
from computation_collective_amd import inputs as gen

pytestmark = pytest.mark.gpu
F32, BF16 = 0, 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _relerr(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert not np.isnan(g).any(), "unwritten (NaN) elements"
    return float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-30))


# the first call: full 256 x 256 tiles (direct-to-LDS mainloop, band folded in
# the mainloop), 8 shards; the second: a smaller, ragged problem (register-
# staged mainloop), 3 shards, 128 x 128 tiles
CALLS = [(8, 512, 1024, 512, BF16, F32, BF16, 256), (3, 300, 328, 136, BF16, BF16, BF16, 128)]


def test_gemm_rs_noalloc_matches_gemm_rs_on_consecutive_calls():
    for k, (P, Mc, N, K, ind, sdt, odt, tm) in enumerate(CALLS):
        print(f"\n[case] noalloc call {k}: P={P} Mc={Mc} N={N} K={K} slot={sdt} tile={tm}", flush=True)
        M = P * Mc
        A, W = gen.gemm_rs_inputs(P, M, N, K, ind, seed=40 + k)
        ref = bf.GemmRS(P, M, N, K, ind, sdt, odt, tm, tm, A, W)
        na = bf.GemmRS(P, M, N, K, ind, sdt, odt, tm, tm, ref.A, ref.W, noalloc=True)
        ref.poison()
        na.poison()
        ref.run()
        na.run()
        torch.cuda.synchronize()
        assert ref.status_value() == 0 and na.status_value() == 0
        assert torch.equal(na.out, ref.out), "output bits differ from hocf_gemm_rs"
        assert torch.equal(na.win_data, ref.win_data), "published slots differ from hocf_gemm_rs"
        assert torch.all(na.win_flags == na.epoch)
        slots, out = oracle.gemm_rs(P, M, N, K, ind, sdt, odt, A, W)
        g = gen.bf16_decode(bf.to_host(na.out, odt)) if odt == BF16 else bf.to_host(na.out, odt)
        o = gen.bf16_decode(out) if odt == BF16 else out
        assert _relerr(g, o) <= 2e-2


def test_gemm_rs_noalloc_rejects_a_workspace_and_oversize():
    # a caller workspace is refused; a problem whose scheduler words exceed the scratch too
    P, M, N, K = 2, 512, 256, 128
    A, W = gen.gemm_rs_inputs(P, M, N, K, BF16, seed=1)
    r = bf.GemmRS(P, M, N, K, BF16, F32, BF16, 256, 256, A, W)
    s = r.next_sync()
    st = hocf.hocf_gemm_rs_noalloc(P, M, N, K, BF16, F32, BF16, r.A, r.W, r.win, r.out, 256, 256, s)
    assert st == hocf.HOCF_ERR_INVALID_ARG
    need = hocf.hocf_gemm_rs_workspace_bytes(16, 16 * 128 * 64, 128 * 64, 128, 128)
    assert need > hocf.HOCF_NOALLOC_SCRATCH_BYTES
