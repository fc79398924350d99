"""Summaries of rocprofv3 CSV output for the profiles/ folder, and the
reader bench.py uses for the HBM traffic figures.

  python -m computation_collective_amd.profsum STATS_DIR FETCH_DIR WRITE_DIR OUT_DIR \\
         "STATS_COMMAND" "COUNTER_COMMAND" [MFMA_DIR "MFMA_COMMAND"]

reads a `rocprofv3 --kernel-trace --stats --output-format csv` run and two
`rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs (COUNTER_COMMAND has
the word COUNTER where the counter name goes) of bench.py -- and, if given,
a run with `--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
GRBM_GUI_ACTIVE` -- and writes one summary per operator,
`OUT_DIR/<workload>.txt`:

  * the kernel's call count and average / min / max duration;
  * FETCH_SIZE and WRITE_SIZE in KiB per dispatch (median over dispatches),
    the same counters for the 1 GiB calibration pass (a negating copy that
    reads and writes 1 GiB), the factors known/measured they give, and the
    scaled bytes per launch between the L2s and the memory fabric (which the
    Infinity Cache may partly serve);
  * the hash of the library sources the counters were taken with, and the
    variant (slot dtype, tile) that was profiled;
  * with the MFMA run: matrix-core busy cycles summed over all SIMDs,
    GRBM_GUI_ACTIVE (reported summed over the 8 XCDs, so divided by 8 for
    one XCD's busy cycles), the MFMA utilisation busy / (XCD cycles *
    SIMDs), the bf16 MFMA flops the kernel issued (MOPS * 512), and, for
    dispatches of 100 us or more, the clock it ran at (XCD cycles / the
    dispatch's counter window).

  python -m computation_collective_amd.profsum copies TRACE_DIR OUT_FILE "COMMAND" "TITLE"

summarises a `rocprofv3 --kernel-trace --memory-copy-trace --stats` run of
bench.py's put operators: the kernels that ran (the runtime's copy kernels
among them) and the copies the copy engines ran.

`traffic(op, variant)` returns the scaled bytes, or None when there is no
summary, it was taken for another variant, or the sources have changed.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import os
import statistics
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30  # the calibration pass reads and writes 1 GiB

# kernel-name fragment -> operator name used by bench.py
KERNELS = [("gemm_rs_kernel<hocf::TileF32", "gemm_rs_tiny"), ("gemm_rs_kernel", "gemm_rs"), ("gemm_ar_kernel", "gemm_ar"), ("gemm_a2a_kernel", "gemm_a2a"),
           ("unfused_gemm_kernel", "gemm_rs_unfused_gemm"), ("unfused_fold_kernel", "gemm_rs_unfused_fold"),
           ("unfused_gemv_kernel", "gemv_ar_unfused_gemv"), ("unfused_gemv_fold_kernel", "gemv_ar_unfused_fold"), ("gemv_ar_kernel", "gemv_ar"),
           ("ag_gemm_kernel", "ag_gemm"), ("embbag_kernel", "embbag_a2a"),
           ("a2a_gemm_kernel<hocf::TileBf16Direct<256, 256, 2, 2, 32, 4>, 1, true, true>", "a2a_gemm"),
           ("a2a_gemm_kernel<hocf::TileBf16Direct<256, 256, 2, 2, 32, 4>, 1, true, false>", "a2a_gemm_unfused_scatter"),
           ("a2a_gemm_kernel<hocf::TileBf16Direct<256, 256, 2, 2, 32, 4>, 1, false, true>", "a2a_gemm_unfused_gemm"),
           ("neg_kernel", "copy")]


def workloads():
    """operator -> (workload name, variant key) of bench.py's default run."""
    from . import configs as c
    return {
        "gemm_rs": (c.GEMM_RS_MLP.name, f"slot_dtype=f32 tile={c.GEMM_RS_MLP.tile_m}x{c.GEMM_RS_MLP.tile_n}"),
        "gemm_rs_tiny": (c.GEMM_RS_TINY.name, f"tile={c.GEMM_RS_TINY.tile_m}x{c.GEMM_RS_TINY.tile_n}"),
        "gemm_rs_unfused_gemm": (c.GEMM_RS_MLP.name + "_unfused_gemm",
                                 f"slot_dtype=f32 tile={c.GEMM_RS_MLP.tile_m}x{c.GEMM_RS_MLP.tile_n}"),
        "gemm_rs_unfused_fold": (c.GEMM_RS_MLP.name + "_unfused_fold",
                                 f"slot_dtype=f32 tile={c.GEMM_RS_MLP.tile_m}x{c.GEMM_RS_MLP.tile_n}"),
        "gemv_ar_unfused_gemv": (c.GEMV_AR_DECODE.name + "_unfused_gemv",
                                 f"tile_n={c.GEMV_AR_DECODE.tile_n} weight_replicas=4"),
        "gemv_ar_unfused_fold": (c.GEMV_AR_DECODE.name + "_unfused_fold",
                                 f"tile_n={c.GEMV_AR_DECODE.tile_n} weight_replicas=4"),
        "gemm_a2a": (c.GEMM_A2A_MOE.name, f"tile={c.GEMM_A2A_MOE.tile_m}x{c.GEMM_A2A_MOE.tile_n}"),
        "gemm_ar": (c.GEMM_AR_MLP.name, f"slot_dtype=f32 tile={c.GEMM_AR_MLP.tile_m}x{c.GEMM_AR_MLP.tile_n}"),
        "gemv_ar": (c.GEMV_AR_DECODE.name, f"tile_n={c.GEMV_AR_DECODE.tile_n} weight_replicas=4"),
        "ag_gemm": (c.AG_GEMM_COL.name, f"tile={c.AG_GEMM_COL.tile_m}x{c.AG_GEMM_COL.tile_n} prereleased"),
        "embbag_a2a": (c.EMBBAG_DLRM.name, f"tile_bags={c.EMBBAG_DLRM.tile_bags}"),
        "a2a_gemm": (c.A2A_GEMM_MOE.name, f"tile={c.A2A_GEMM_MOE.tile_m}x{c.A2A_GEMM_MOE.tile_n}"),
        "a2a_gemm_unfused_scatter": (c.A2A_GEMM_MOE.name + "_unfused_scatter",
                                     f"tile={c.A2A_GEMM_MOE.tile_m}x{c.A2A_GEMM_MOE.tile_n}"),
        "a2a_gemm_unfused_gemm": (c.A2A_GEMM_MOE.name + "_unfused_gemm",
                                  f"tile={c.A2A_GEMM_MOE.tile_m}x{c.A2A_GEMM_MOE.tile_n}"),
    }


def source_hash() -> str:
    """sha256 over the library's HIP/C++ sources and the ABI header."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*"))) + [os.path.join(ROOT, "include", "hocf.h")]
    for f in files:
        if os.path.isfile(f):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def op_of(kernel_name: str):
    for frag, op in KERNELS:
        if frag in kernel_name:
            return op
    return None


def _find_csv(path: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {path}")
    return hits[0]


SIMDS = 256 * 4  # MI355X: 256 CUs of 4 SIMDs
XCDS = 8


def counter_medians(path: str, counter: str) -> dict:
    """op -> median over dispatches of the counter summed over its instances."""
    per = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(_find_csv(path, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        op = op_of(r["Kernel_Name"])
        if op:
            per[op][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {op: statistics.median(d.values()) for op, d in per.items()}


def counter_windows_us(path: str, counter: str) -> dict:
    """op -> median over dispatches of the counter row's own time window."""
    per = defaultdict(list)
    for r in csv.DictReader(open(_find_csv(path, "counter_collection.csv"))):
        op = op_of(r["Kernel_Name"])
        if r["Counter_Name"] == counter and op:
            per[op].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {op: statistics.median(v) for op, v in per.items()}


def kernel_stats(path: str) -> dict:
    out = {}
    for r in csv.DictReader(open(_find_csv(path, "kernel_stats.csv"))):
        op = op_of(r["Name"])
        if op and op not in out:
            out[op] = (r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                       float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3)
    return out


def summarize(stats_dir, fetch_dir, write_dir, out_dir, stats_cmd, counter_cmd, mfma_dir=None,
              mfma_cmd=None) -> None:
    stats = kernel_stats(stats_dir)
    fetch = counter_medians(fetch_dir, "FETCH_SIZE")
    write = counter_medians(write_dir, "WRITE_SIZE")
    busy = counter_medians(mfma_dir, "SQ_VALU_MFMA_BUSY_CYCLES") if mfma_dir else {}
    mops = counter_medians(mfma_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16") if mfma_dir else {}
    active = counter_medians(mfma_dir, "GRBM_GUI_ACTIVE") if mfma_dir else {}
    window = counter_windows_us(mfma_dir, "GRBM_GUI_ACTIVE") if mfma_dir else {}
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("the calibration pass is missing from the counter runs")
    ff = COPY_BYTES / 1024.0 / fetch["copy"]
    fw = COPY_BYTES / 1024.0 / write["copy"]
    src = source_hash()
    os.makedirs(out_dir, exist_ok=True)
    for op, (wl, variant) in workloads().items():
        if op not in stats:
            continue
        name, calls, avg, mn, mx = stats[op]
        lines = [f"# rocprofv3 summary: {op} kernel, workload {wl}",
                 f"# kernel statistics: {stats_cmd}",
                 f"# counters (one run per counter): {counter_cmd}",
                 f"# calibration: a 1 GiB negating copy in the same runs reads FETCH_SIZE {fetch['copy']:.0f} KiB"
                 f" and WRITE_SIZE {write['copy']:.0f} KiB for 1048576 KiB each"]
        if mfma_cmd:
            lines.append(f"# matrix cores: {mfma_cmd}")
        lines += [
                 f"kernel {name}",
                 f"variant {variant}",
                 f"sources {src}",
                 f"stats calls={calls} avg_us={avg:.2f} min_us={mn:.2f} max_us={mx:.2f}"]
        if op in fetch and op in write:
            # (FETCH_SIZE / WRITE_SIZE count traffic between the L2s and the memory fabric; the
            # Infinity Cache behind the fabric may serve part of it, so it is an upper bound of
            # the DRAM traffic, not a DRAM-side count)
            b = fetch[op] * 1024 * ff + write[op] * 1024 * fw
            lines.append(f"counters fetch_kib={fetch[op]:.0f} write_kib={write[op]:.0f} "
                         f"fetch_factor={ff:.4f} write_factor={fw:.4f} l2_fabric_bytes={b:.0f}")
        if op in busy and op in active and active[op] > 0:
            xcd_cycles = active[op] / XCDS
            util = busy[op] / (xcd_cycles * SIMDS)
            line = (f"mfma busy_cycles={busy[op]:.0f} gui_active_cycles={active[op]:.0f} xcds={XCDS} "
                    f"simds={SIMDS} util={util:.4f} bf16_flops={mops.get(op, 0) * 512:.0f} "
                    f"window_us={window[op]:.1f}")
            # the clock only for long dispatches: a fixed overhead of some 20 k cycles per dispatch
            # in the counter window makes it meaningless below ~100 us
            if avg >= 100.0:
                line += f" clock_mhz={xcd_cycles / window[op]:.0f}"
            lines.append(line)
        with open(os.path.join(out_dir, wl + ".txt"), "w") as fh:
            fh.write("\n".join(lines) + "\n")


def _fields(path):
    d = {}
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        key, _, rest = line.rstrip("\n").partition(" ")
        d[key] = rest
    return d


# bench operators whose timed call launches several kernels
COMPOSITE = {"gemm_rs_unfused": ("gemm_rs_unfused_gemm", "gemm_rs_unfused_fold"),
             "a2a_gemm_unfused": ("a2a_gemm_unfused_scatter", "a2a_gemm_unfused_gemm"),
             "gemv_ar_unfused": ("gemv_ar_unfused_gemv", "gemv_ar_unfused_fold")}


def traffic(op: str, variant: str | None = None):
    """Scaled HBM bytes per launch of `op` from its committed summary, or None
    when there is none, it covers another variant, or the sources changed
    (for an operator of several kernels: their sum, if every one is known)."""
    if op in COMPOSITE:
        parts = [traffic(k, variant) for k in COMPOSITE[op]]
        return None if any(x is None for x in parts) else float(sum(parts))
    wl = workloads().get(op)
    if wl is None:
        return None
    path = os.path.join(PROFILES, wl[0] + ".txt")
    if not os.path.isfile(path):
        return None
    d = _fields(path)
    if d.get("sources") != source_hash() or d.get("variant") != (variant or wl[1]) or "counters" not in d:
        return None
    kv = dict(x.split("=") for x in d["counters"].split())
    return float(kv["l2_fabric_bytes"]) if "l2_fabric_bytes" in kv else None


def summarize_copies(trace_dir, out_file, command, title) -> None:
    """Summary of a `rocprofv3 --kernel-trace --memory-copy-trace --stats` run
    of bench.py's put operators: every kernel with its call count and average
    duration (the runtime's copy kernels among them), and every kind of memory
    copy the copy engines ran.  Host-to-device copies are the upload of the
    inputs before the timed steps."""
    lines = [f"# rocprofv3 summary: {title}", f"# command: {command}",
             f"sources {source_hash()}", "kernels (name, calls, avg_us, total_us)"]
    for r in csv.DictReader(open(_find_csv(trace_dir, "kernel_stats.csv"))):
        name = r["Name"]
        short = name if len(name) <= 90 else name[:87] + "..."
        lines.append(f"  {short} calls={r['Calls']} avg_us={float(r['AverageNs']) / 1e3:.2f} "
                     f"total_us={float(r['TotalDurationNs']) / 1e3:.1f}")
    lines.append("copy-engine copies (direction, calls, avg_us, min_us, max_us, total_us)")
    for r in csv.DictReader(open(_find_csv(trace_dir, "memory_copy_stats.csv"))):
        lines.append(f"  {r['Name']} calls={r['Calls']} avg_us={float(r['AverageNs']) / 1e3:.2f} "
                     f"min_us={float(r['MinNs']) / 1e3:.2f} max_us={float(r['MaxNs']) / 1e3:.2f} "
                     f"total_us={float(r['TotalDurationNs']) / 1e3:.1f}")
    with open(out_file, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if len(sys.argv) == 6 and sys.argv[1] == "copies":
        summarize_copies(*sys.argv[2:])
    elif len(sys.argv) in (7, 9):
        summarize(*sys.argv[1:])
    else:
        raise SystemExit(__doc__)
