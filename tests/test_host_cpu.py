"""Host logic of the measurement tools, on hand-built inputs (CPU only):

* profsum: kernel names -> operators; the counter summaries (calibration on
  the 1 GiB copy, medians over dispatches, matrix-core utilisation, the
  clock only for long dispatches); `traffic()` trusting a summary only for
  the current sources and the profiled variant;
* bench.py: a multi-GPU request ends with a message, before any GPU work.
"""

import csv
import os
import subprocess
import sys

import pytest

from computation_collective_amd import configs as cfgs
from computation_collective_amd import profsum

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RS_KERNEL = "void hocf::gemm_rs_kernel<hocf::TileBf16Direct<256, 256, 2, 2, 32, 4>, false, true, 0, 1>(hocf::GemmRsArgs)"
TINY_KERNEL = "void hocf::gemm_rs_kernel<hocf::TileF32<64, 64, 2, 2>, false, false, 0, 0>(hocf::GemmRsArgs)"
COPY_KERNEL = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"


def test_op_of_maps_kernel_names():
    assert profsum.op_of(RS_KERNEL) == "gemm_rs"
    assert profsum.op_of(TINY_KERNEL) == "gemm_rs_tiny"
    assert profsum.op_of("void hocf::gemm_ar_kernel<x>(hocf::GemmRsArgs)") == "gemm_ar"
    assert profsum.op_of("void hocf::unfused_gemm_kernel<x>(a)") == "gemm_rs_unfused_gemm"
    assert profsum.op_of("void hocf::unfused_fold_kernel<x>(a)") == "gemm_rs_unfused_fold"
    assert profsum.op_of("void hocf::unfused_gemv_kernel<4, 256, 0, 1>(a)") == "gemv_ar_unfused_gemv"
    assert profsum.op_of("void hocf::unfused_gemv_fold_kernel<4, 256, 0, 1>(a)") == "gemv_ar_unfused_fold"
    assert profsum.op_of("void hocf::gemv_ar_kernel<4, 256, 0, 1>(a)") == "gemv_ar"
    assert profsum.op_of(COPY_KERNEL) == "copy"
    assert profsum.op_of("__amd_rocclr_copyBuffer") is None


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _counter_rows(counter, per_kernel):
    """per_kernel: [(kernel name, dispatch id, [instance values], window ns)]"""
    rows = []
    for name, disp, vals, ns in per_kernel:
        for v in vals:
            rows.append(dict(Counter_Name=counter, Kernel_Name=name, Dispatch_Id=disp, Counter_Value=v,
                             Start_Timestamp=1000, End_Timestamp=1000 + ns))
    return rows


def test_summarize_calibrates_on_the_copy(tmp_path):
    # the copy reads FETCH_SIZE 524288 KiB and WRITE_SIZE 1048576 KiB for its 1 GiB each way:
    # factors 2 and 1.  gemm_rs: two dispatches, counters summed over two instances each, the
    # median over dispatches taken.
    st, fe, wr, mf, out = (str(tmp_path / n) for n in ("stats", "fetch", "write", "mfma", "out"))
    _write_csv(os.path.join(st, "s_kernel_stats.csv"), [
        dict(Name=RS_KERNEL, Calls=12, AverageNs=1000000, MinNs=990000, MaxNs=1100000),
        dict(Name=TINY_KERNEL, Calls=12, AverageNs=28000, MinNs=27000, MaxNs=31000)])
    _write_csv(os.path.join(fe, "f_counter_collection.csv"), _counter_rows("FETCH_SIZE", [
        (COPY_KERNEL, 1, [262144, 262144], 100000),
        (RS_KERNEL, 2, [400, 600], 1000000), (RS_KERNEL, 3, [500, 700], 1000000),
        (RS_KERNEL, 4, [9000, 9000], 1000000)]))
    _write_csv(os.path.join(wr, "w_counter_collection.csv"), _counter_rows("WRITE_SIZE", [
        (COPY_KERNEL, 1, [1048576], 100000), (RS_KERNEL, 2, [500], 1000000)]))
    # a 1 ms dispatch: 2e6 cycles of each XCD (2 GHz), half of them busy on every SIMD
    mrows = (_counter_rows("SQ_VALU_MFMA_BUSY_CYCLES", [(RS_KERNEL, 5, [1024 * 1000000], 1000000),
                                                        (TINY_KERNEL, 6, [1024], 28000)]) +
             _counter_rows("SQ_INSTS_VALU_MFMA_MOPS_BF16", [(RS_KERNEL, 5, [1000], 1000000)]) +
             _counter_rows("GRBM_GUI_ACTIVE", [(RS_KERNEL, 5, [8 * 2000000], 1000000),
                                               (TINY_KERNEL, 6, [8 * 100], 28000)]))
    _write_csv(os.path.join(mf, "m_counter_collection.csv"), mrows)
    profsum.summarize(st, fe, wr, out, "STATS CMD", "COUNTER CMD", mf, "MFMA CMD")
    rs = profsum._fields(os.path.join(out, cfgs.GEMM_RS_MLP.name + ".txt"))
    assert rs["sources"] == profsum.source_hash()
    assert rs["stats"] == "calls=12 avg_us=1000.00 min_us=990.00 max_us=1100.00"
    c = dict(kv.split("=") for kv in rs["counters"].split())
    assert c["fetch_kib"] == "1200" and c["write_kib"] == "500"      # median of 1000, 1200, 18000
    assert float(c["fetch_factor"]) == pytest.approx(2.0) and float(c["write_factor"]) == pytest.approx(1.0)
    assert int(c["l2_fabric_bytes"]) == 1200 * 1024 * 2 + 500 * 1024
    m = dict(kv.split("=") for kv in rs["mfma"].split())
    assert float(m["util"]) == pytest.approx(0.5)
    assert int(m["bf16_flops"]) == 1000 * 512
    assert m["clock_mhz"] == "2000"                                    # 2e6 cycles in a 1 ms window
    tiny = profsum._fields(os.path.join(out, cfgs.GEMM_RS_TINY.name + ".txt"))
    assert "counters" not in tiny                                      # not in the counter runs
    assert "clock_mhz" not in tiny["mfma"]                             # a 28 us dispatch: no clock


def test_summarize_needs_the_calibration(tmp_path):
    st, fe, wr = (str(tmp_path / n) for n in ("stats", "fetch", "write"))
    _write_csv(os.path.join(st, "s_kernel_stats.csv"),
               [dict(Name=RS_KERNEL, Calls=1, AverageNs=1, MinNs=1, MaxNs=1)])
    for d, ctr in ((fe, "FETCH_SIZE"), (wr, "WRITE_SIZE")):
        _write_csv(os.path.join(d, "c_counter_collection.csv"), _counter_rows(ctr, [(RS_KERNEL, 1, [1], 1)]))
    with pytest.raises(SystemExit):
        profsum.summarize(st, fe, wr, str(tmp_path / "out"), "a", "b")


def _summary(path, op, sources, variant, l2):
    wl = profsum.workloads()[op][0]
    with open(os.path.join(path, wl + ".txt"), "w") as fh:
        fh.write(f"# rocprofv3 summary: {op}\nvariant {variant}\nsources {sources}\n"
                 f"stats calls=1 avg_us=1.00 min_us=1.00 max_us=1.00\n"
                 f"counters fetch_kib=1 write_kib=1 fetch_factor=2.0 write_factor=1.0 l2_fabric_bytes={l2}\n")


def test_traffic_only_for_the_current_sources_and_variant(tmp_path, monkeypatch):
    monkeypatch.setattr(profsum, "PROFILES", str(tmp_path))
    src = profsum.source_hash()
    var = profsum.workloads()["gemm_rs"][1]
    assert profsum.traffic("gemm_rs") is None                          # no summary
    _summary(tmp_path, "gemm_rs", src, var, 123456)
    assert profsum.traffic("gemm_rs") == 123456
    assert profsum.traffic("gemm_rs", "slot_dtype=bf16 tile=256x256") is None   # another variant
    _summary(tmp_path, "gemm_rs", "0000000000000000", var, 123456)
    assert profsum.traffic("gemm_rs") is None                          # other sources
    # an operator of two kernels: the sum, once both are known
    v2 = profsum.workloads()["gemm_rs_unfused_gemm"][1]
    _summary(tmp_path, "gemm_rs_unfused_gemm", src, v2, 1000)
    assert profsum.traffic("gemm_rs_unfused") is None
    _summary(tmp_path, "gemm_rs_unfused_fold", src, v2, 24)
    assert profsum.traffic("gemm_rs_unfused") == 1024


def test_bench_refuses_several_gpus_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
