"""Per-iteration timeline of the fused GEMM + ReduceScatter kernel, from the
library's trace build (libhocf_trace.so, csrc/trace.hpp), and the summary
that sets the rank-order folds against the other workgroups' GEMM work.

The method's claim (SC24 abstract; mKernel, section on persistent kernels
and tile/chunk overlap) is that a workgroup's collective work -- here the
fold of a completed output tile's P published partials -- runs while other
workgroups of the same kernel still compute.  Every iteration of every
workgroup records six timestamps on the device's constant wall clock (the
same clock on every CU): iteration start, claim resolved, mainloop start,
mainloop end, tile stores completed, flag and count done; plus the tile and
the band it took.  From those:

  * fold intervals: a band folded inside a mainloop occupies that mainloop
    [start, end]; a band folded on its own occupies [claim, mainloop start];
  * GEMM intervals: every [mainloop start, mainloop end];
  * overlap: over the total fold time, how many OTHER workgroups were in a
    mainloop (a 0.25 us grid), and the share of fold time during which at
    least one, and at least half of them, were;
  * phases per tile iteration, the drain (from the last mainloop's end to
    the kernel's last record), and each XCD's last mainloop end (the skew
    between XCDs);
  * store contention: during each tile's slot stores, how many other
    workgroups of the same XCD are storing, and the store time by that
    count.

  python -m computation_collective_amd.trace [--calls N] [--slot-dtype f32|bf16] [--out FILE]
                                            [--save-out FILE.npy]

runs the 8-shard 8192 x 4096 x 1792 bf16 workload (tile 256 x 256) N times
on cuda:0 with the trace library and writes the summary of the last call.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# record layout (csrc/trace.hpp)
TRACE_ITERS = 64
TRACE_WGS = 2048
REC_WORDS = 8
TRACE_BYTES = TRACE_ITERS * TRACE_WGS * REC_WORDS * 8
T_START, T_CLAIMED, T_MAIN0, T_MAIN1, T_STORED, T_DONE = range(6)
BIT_IN_LOOP, BIT_ALONE, BIT_COMPLETED = 1, 2, 4
XCDS = 8


def wall_clock_khz(device: int = 0) -> int:
    """The device wall clock's rate (hipDeviceAttributeWallClockRate)."""
    import torch  # noqa: F401  (loads the HIP runtime torch was built with)
    for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
        try:
            hip = ctypes.CDLL(name)
            break
        except OSError:
            continue
    else:
        raise RuntimeError("HIP runtime library not found")
    v = ctypes.c_int(0)
    rc = hip.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(10017), ctypes.c_int(device))
    if rc != 0 or v.value <= 0:
        raise RuntimeError(f"hipDeviceGetAttribute(WallClockRate) failed ({rc})")
    return v.value


def parse(raw: np.ndarray, grid: int):
    """Records -> dict of flat arrays (one entry per recorded iteration)."""
    rec = raw.reshape(TRACE_WGS, TRACE_ITERS, REC_WORDS)[:grid]
    wg, it = np.nonzero(rec[:, :, T_START] != 0)
    r = rec[wg, it]
    band = (r[:, 7] & 0xFFFFFFFF).astype(np.int64)
    band[band == 0xFFFFFFFF] = -1
    return dict(wg=wg, it=it, t=r[:, :6].astype(np.int64), item=r[:, 6].view(np.int64),
                band=band, bits=(r[:, 7] >> 32).astype(np.int64))


def output_tile(item, P: int, mtiles: int, ntiles: int):
    """Work item -> the output tile (chunk r, row tile, column tile) it contributes to, numbered
    r * tiles-per-chunk + row tile * ntiles + column tile (the kernel's item order: shard,
    chunk, then column tile major within a chunk)."""
    tpc = mtiles * ntiles
    tq = item % tpc
    r = item // tpc % P
    return r * tpc + (tq % mtiles) * ntiles + tq // mtiles


def summarize(d, khz: int, P: int, mtiles: int, ntiles: int, pieces: int,
              span_event_us: float | None = None) -> list[str]:
    tpc = mtiles * ntiles
    us = 1e3 / khz                      # microseconds per tick
    t = d["t"]
    t0 = t[:, T_START].min()
    T = (t - t0) * us                   # microseconds from the kernel's first record
    end = T[:, T_DONE].max()
    has_tile = d["item"] >= 0
    in_loop = (d["bits"] & BIT_IN_LOOP) != 0
    alone = (d["bits"] & BIT_ALONE) != 0
    nwg = int(d["wg"].max()) + 1

    lines = []
    lines.append(f"clock wall_clock_khz={khz} tick_us={us:.4f}")
    lines.append(f"span_us={end:.1f}" + (f" event_us={span_event_us:.1f}" if span_event_us else "") +
                 f" workgroups={nwg} iterations={len(T)} tiles={int(has_tile.sum())} "
                 f"bands={int((in_loop | alone).sum())} (expected {P * tpc * pieces}: {pieces} per output tile)")

    # phases of the iterations that computed a tile
    tl = T[has_tile]
    ph = dict(claim=tl[:, T_CLAIMED] - tl[:, T_START],
              prologue_and_lone_band=tl[:, T_MAIN0] - tl[:, T_CLAIMED],
              mainloop_with_band=(tl[:, T_MAIN1] - tl[:, T_MAIN0])[in_loop[has_tile]],
              mainloop_without_band=(tl[:, T_MAIN1] - tl[:, T_MAIN0])[~in_loop[has_tile]],
              store=tl[:, T_STORED] - tl[:, T_MAIN1],
              flag_and_count=tl[:, T_DONE] - tl[:, T_STORED])
    lines.append("phase_us (tile iterations: mean, p10, p90, count) " + " ".join(
        f"{k}={v.mean():.2f},{np.percentile(v, 10):.2f},{np.percentile(v, 90):.2f},{len(v)}"
        for k, v in ph.items() if len(v)))
    per_wg_tiles = np.bincount(d["wg"][has_tile], minlength=nwg)
    per_wg_busy = np.zeros(nwg)
    np.add.at(per_wg_busy, d["wg"][has_tile], tl[:, T_MAIN1] - tl[:, T_MAIN0])
    lines.append(f"per_workgroup tiles_min={per_wg_tiles.min()} tiles_max={per_wg_tiles.max()} "
                 f"mainloop_share_of_span={per_wg_busy.mean() / end:.3f}")

    # GEMM intervals on a 0.25 us grid: how many workgroups are in a mainloop
    step = 0.25
    nb = int(np.ceil(end / step)) + 1
    cover = np.zeros(nb + 1)
    g0 = np.floor(tl[:, T_MAIN0] / step).astype(np.int64)
    g1 = np.floor(tl[:, T_MAIN1] / step).astype(np.int64)
    np.add.at(cover, g0, 1)
    np.add.at(cover, g1, -1)
    active = np.cumsum(cover)[:nb]

    # fold intervals, with the folding workgroup's own mainloop taken out
    folds = []
    for k in np.nonzero(in_loop | alone)[0]:
        if in_loop[k]:
            a, b, own = T[k, T_MAIN0], T[k, T_MAIN1], 1
        else:
            a, b, own = T[k, T_CLAIMED], T[k, T_MAIN0], 0
        folds.append((a, b, own))
    tot = other_sum = ge1 = gehalf = 0.0
    for a, b, own in folds:
        i0, i1 = int(a / step), max(int(b / step), int(a / step) + 1)
        seg = active[i0:i1] - own
        tot += len(seg)
        other_sum += seg.sum()
        ge1 += (seg >= 1).sum()
        gehalf += (seg >= (nwg - 1) / 2).sum()
    lines.append(f"folds in_mainloop={int(in_loop.sum())} alone={int(alone.sum())} "
                 f"alone_with_a_tile={int((alone & has_tile).sum())} alone_without_tile={int((alone & ~has_tile).sum())}")
    if tot:
        lines.append(f"overlap fold_time_us={tot * step:.1f} mean_other_workgroups_in_mainloop={other_sum / tot:.1f} "
                     f"of={nwg - 1} share_with_one_or_more_other={ge1 / tot:.3f} "
                     f"share_with_half_or_more={gehalf / tot:.3f}")

    # when each band is folded relative to the GEMM work
    last_main = tl[:, T_MAIN1].max()
    fold_end = np.array([b for _, b, _ in folds])
    lines.append(f"bands_folded_before_last_mainloop_end={np.mean(fold_end <= last_main):.3f} "
                 f"drain_us={end - last_main:.1f}")

    # output tile ready (its last producer's flag and count) -> band folded
    done = has_tile & ((d["bits"] & BIT_COMPLETED) != 0)
    grp = output_tile(d["item"][done], P, mtiles, ntiles)
    ready = dict(zip(grp.tolist(), T[done, T_DONE].tolist()))
    lat = []
    for k in np.nonzero(in_loop | alone)[0]:
        g = int(d["band"][k]) // pieces
        if g in ready:
            lat.append((T[k, T_MAIN1] if in_loop[k] else T[k, T_MAIN0]) - ready[g])
    if lat:
        lat = np.array(lat)
        lines.append(f"ready_to_folded_us median={np.median(lat):.1f} p90={np.percentile(lat, 90):.1f} "
                     f"max={lat.max():.1f} output_tiles_completed={len(ready)}")

    # slot-store contention: while a workgroup stores its tile, how many other
    # workgroups of its XCD store theirs (all of an XCD's stores leave through
    # that XCD's L2), and the store time against that count
    xcd = d["wg"][has_tile] % XCDS
    s0, s1 = tl[:, T_MAIN1], tl[:, T_STORED]
    same = np.zeros(len(tl))
    for x in range(XCDS):
        m = np.nonzero(xcd == x)[0]
        if len(m) == 0:
            continue
        c = np.zeros(nb + 1)
        np.add.at(c, np.floor(s0[m] / step).astype(np.int64), 1)
        np.add.at(c, np.floor(s1[m] / step).astype(np.int64), -1)
        storing = np.cumsum(c)[:nb]
        for k in m:
            i0 = int(s0[k] / step)
            i1 = max(int(s1[k] / step), i0 + 1)
            same[k] = storing[i0:i1].mean() - 1
    dur = s1 - s0
    buckets = []
    for lo, hi in ((0, 8), (8, 16), (16, 24), (24, 10 ** 9)):
        m = (same >= lo) & (same < hi)
        if m.any():
            buckets.append(f"{lo}-{hi - 1 if hi < 10 ** 9 else 'up'}:{dur[m].mean():.2f},{int(m.sum())}")
    lines.append(f"store_contention same_xcd_others_storing_mean={same.mean():.1f} "
                 f"store_us_by_others_storing(mean,count)=" + " ".join(buckets))

    # skew between XCDs (workgroups are dispatched round-robin: XCD = index mod 8)
    lastx = np.array([tl[xcd == x, T_MAIN1].max() for x in range(XCDS) if np.any(xcd == x)])
    lines.append("xcd_last_mainloop_end_us " + " ".join(f"{v:.1f}" for v in lastx) +
                 f" spread={lastx.max() - lastx.min():.1f}")
    return lines


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--calls", type=int, default=3)
    ap.add_argument("--slot-dtype", choices=["f32", "bf16"], default="f32")
    ap.add_argument("--out", default=None)
    ap.add_argument("--save-out", default=None, help="also save the last call's output tensor (.npy)")
    args = ap.parse_args(argv)

    sys.path.insert(0, ROOT)
    import torch

    from computation_collective_amd import buffers as bf
    from computation_collective_amd import configs as cfgs
    from computation_collective_amd import hocf
    from computation_collective_amd import inputs as gen

    hocf.use_trace_library()
    torch.cuda.set_device(0)
    c = cfgs.GEMM_RS_MLP
    sdt = bf.F32 if args.slot_dtype == "f32" else bf.BF16
    A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, c.in_dt, seed=0)
    run = bf.GemmRS(c.P, c.M, c.N, c.K, c.in_dt, sdt, c.out_dt, c.tile_m, c.tile_n, A, W)
    del A, W
    ws_bytes = hocf.hocf_gemm_rs_workspace_bytes(c.P, c.M, c.N, c.tile_m, c.tile_n)
    off = ws_bytes - TRACE_BYTES
    assert off > 0 and off % 256 == 0, "not the trace build's workspace"
    region = run.ws.view(torch.uint8)[off:off + TRACE_BYTES]
    khz = wall_clock_khz()
    stream = torch.cuda.Stream()
    raw = None
    ev_us = None
    for k in range(args.calls):
        region.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            run.run(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        if run.status_value() != 0:
            raise SystemExit(f"device status {run.status_value()}")
        ev_us = e0.elapsed_time(e1) * 1e3
        raw = region.cpu().numpy().view(np.uint64)
        print(f"[trace] call {k}: {ev_us:.1f} us", flush=True)
    mtiles, ntiles = c.M // c.P // c.tile_m, c.N // c.tile_n
    pieces = 8   # bands per 256 x 256 tile (32 rows each)
    d = parse(raw, TRACE_WGS)
    grid = int(d["wg"].max()) + 1
    lines = [f"# trace summary: gemm_rs kernel (trace build), workload {c.name}, slot_dtype={args.slot_dtype}",
             f"# command: python -m computation_collective_amd.trace --calls {args.calls} "
             f"--slot-dtype {args.slot_dtype}" + (f" --out {args.out}" if args.out else ""),
             f"# figures of the last of {args.calls} calls; times in microseconds from the kernel's first record",
             f"grid {grid}"]
    lines += summarize(d, khz, c.P, mtiles, ntiles, pieces, span_event_us=ev_us)
    text = "\n".join(lines) + "\n"
    print(text, flush=True)
    if args.save_out:
        np.save(args.save_out, run.out.cpu().numpy())
    if args.out:
        os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
        with open(args.out, "w") as f:
            f.write(text)
        np.save(os.path.splitext(args.out)[0] + "_records.npy", raw.reshape(TRACE_WGS, TRACE_ITERS, REC_WORDS)[:grid])


if __name__ == "__main__":
    main()
