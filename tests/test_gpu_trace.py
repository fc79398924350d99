"""The trace build of the GEMM + ReduceScatter kernel (libhocf_trace.so: six
wall-clock stamps per iteration of every workgroup, written to a workspace
extension) on the MLP-down workload.  The stamps must change nothing the
kernel computes: its output is bit-identical to the product library's on
the same inputs, and every tile and every band of the call is recorded.

The trace library cannot be loaded beside the product library in one
process, so it runs in a child process (computation_collective_amd.trace).
"""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from computation_collective_amd import buffers as bf
from computation_collective_amd import configs as cfgs
from computation_collective_amd import hocf
from computation_collective_amd import inputs as gen

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_trace_build_output_identical_and_every_iteration_recorded(tmp_path):
    assert os.path.exists(hocf.TRACE_LIB_PATH), "libhocf_trace.so is not built"
    c = cfgs.GEMM_RS_MLP
    summary, out_npy = tmp_path / "summary.txt", tmp_path / "out.npy"
    print(f"[case] trace build, {c.name}, child process", flush=True)
    r = subprocess.run([sys.executable, "-m", "computation_collective_amd.trace", "--calls", "1",
                        "--out", str(summary), "--save-out", str(out_npy)],
                       cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    text = summary.read_text()
    tiles = c.P * (c.M // c.tile_m) * (c.N // c.tile_n)
    assert f"tiles={tiles} bands={tiles}" in text, text  # 8 bands per output tile, P tiles per output tile

    print("[case] product library, same inputs", flush=True)
    A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, c.in_dt, seed=0)
    run = bf.GemmRS(c.P, c.M, c.N, c.K, c.in_dt, c.slot_dt, c.out_dt, c.tile_m, c.tile_n, A, W)
    run.run()
    torch.cuda.synchronize()
    assert run.status_value() == 0
    assert np.array_equal(run.out.cpu().numpy(), np.load(out_npy))
