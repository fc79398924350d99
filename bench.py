#!/usr/bin/env python3
"""Bench of the fused computation + collective-epilogue hot path on one MI355X.

One step = one pass of the whole hot path: one call of each fused operator
at its workload size, on one HIP stream, inputs already resident in HBM:

  gemm_rs     GEMM+ReduceScatter, P=8, A_p 8192x1792, W_p 1792x4096 bf16, tile 256x256
  gemm_rs_tiny  GEMM+ReduceScatter, P=4, A_p and W_p 256x256 fp32 U[-1,1), tile 64x64 (the fp32
              matrix-core path; its roofline is the fp32 MFMA peak, its time is launch-bound)
  gemv_ar     GEMV+AllReduce, P=8, x_p 4x1024, W_p 1024x8192 bf16 (4 weight replicas rotate;
              a 1 GiB scratch read before each call, outside the timed events)
  ag_gemm     AllGather+GEMM, 8 chunks 1024x4096, W 4096x1792 bf16, chunk flags written in a
              seeded random order on the kernel's stream just before it (outside the timed
              events: the kernel's span is timed)
  ag_gemm_paced  the same with the chunks arriving over time, as over xGMI: the host sets
              the flags (host-coherent memory) 55 us apart after the launch (--chunk-gap-us);
              after_last_arrival_us = the kernel's span minus the 385 us arrival span
  embbag_a2a  64 tables 1e6x128 fp32, batch 16384, 20 rows per bag, Zipf(1.05), P=8
              (a 1 GiB scratch read before each call, outside the timed events); its roofline
              counts the compulsory bytes (every distinct row once, the indices, the pooled
              rows written), which no gather can go below; `logical_gbps` counts every
              looked-up row (Zipf repeats included, served mostly by the caches)
  gemm_ar     GEMM+AllReduce, the gemm_rs shapes; the folded chunks land in all 8 windows
  gemm_a2a    GEMM+All-to-All (MoE combine): 8 ranks x 4096 tokens, top-2 of 32 experts, this
              rank's 4 experts 1792 -> 4096 bf16, each result row sent to its token's rank
  a2a_gemm    All-to-All+GEMM (MoE dispatch): the same routing; the rows chosen for this rank's 4
              experts are counted, placed and delivered on the device, grouped by expert, and
              projected 4096 -> 1792 bf16 as their row tiles complete
  gemm_rs_unfused, gemv_ar_unfused  the gemm_rs / gemv_ar workloads as two kernels (the
              computation publishing its partials, then the fold): the bulk-synchronous
              baseline; `fusion` reports the time each fused operator saves against it
  a2a_gemm_unfused  the dispatch delivering every row, then the expert GEMM (two kernels)
  gemm_rs_decomp<d>_f<F>  Compass's inter-operator decomposition on one GPU: the gemm_rs workload
              as d column pieces, each piece's GEMM on the step's stream with F CUs left free, its
              fold on a second stream overlapping the next piece's GEMM; `fusion.gemm_rs` lists them

ag_gemm_dma, ag_gemm_cu_put  the ag_gemm workload with its seven remote chunks delivered during
              the call by hocf_dma_put on a second stream (HOCCL's copy-engine communication):
              on the copy (SDMA) engines, no compute unit, or on the runtime's copy kernels
              (each chunk signalled by its flag)
dma_put, cu_put  those seven 8 MB puts alone, unsignalled (ordered by the streams alone; GB/s
              counts each byte read and written)
gemm_rs_dma_put, gemm_rs_cu_put  the gemm_rs workload with the same unsignalled puts enqueued just
              before it on a second stream: what communication on the copy engines, or on the
              compute units, costs a kernel that holds every CU

hipblaslt_bmm: context, not an operator of this library -- torch.bmm (hipBLASLt) on the same
eight shard GEMMs as gemm_rs, with no collective.

Optional extra ops (--ops): embbag_uniform (the same shapes with uniform indices:
no reuse, a control for the Zipf figure) and copy (a 1 GiB negating copy, the
calibration of the HBM byte counters).

`value` is the GEMM+ReduceScatter throughput (TFLOP/s, the headline kernel);
each operator's own throughput and roofline fraction are in `ops`.  Each
kernel's time comes from HIP events recorded on the stream it runs on.

  python bench.py [--steps K] [--warmup W] [--slot-dtype f32|bf16] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused GEMM+ReduceScatter TFLOP/s & GEMV/embbag GB/s, % roofline, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CUs x 2.4 GHz x 4096 flop/clock)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)  # >= 200 timed calls of each operator
    ap.add_argument("--warmup", type=int, default=10)  # untimed steps first (10 calls of each operator)
    ap.add_argument("--slot-dtype", choices=["f32", "bf16"], default="f32")
    # (each fused operator and its unfused baseline run back to back within a step)
    ap.add_argument("--ops", default="gemm_rs,gemm_rs_unfused,gemv_ar,gemv_ar_unfused,a2a_gemm,a2a_gemm_unfused,"
                                     "gemm_rs_tiny,ag_gemm,ag_gemm_paced,ag_gemm_dma,ag_gemm_cu_put,dma_put,cu_put,"
                                     "gemm_rs_dma_put,gemm_rs_cu_put,embbag_a2a,gemm_ar,gemm_a2a,"
                                     "gemm_rs_decomp2_f32,gemm_rs_decomp4_f32,gemm_rs_decomp8_f32,"
                                     "hipblaslt_bmm")
    ap.add_argument("--gemv-tile", type=int, default=0, help="GEMV column tile (default: the config's)")
    ap.add_argument("--a2a-tile-m", type=int, default=0, help="GEMM+A2A tile rows (default: the config's)")
    ap.add_argument("--chunk-gap-us", type=float, default=55.0,
                    help="ag_gemm_paced: time between chunk arrivals (8 MB over one ~153 GB/s xGMI link)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    return ap.parse_args()


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def cpu_baseline(target_s):
    """The oracle (unchanged) on the host cores, on a bounded sample of the
    GEMM+ReduceScatter workload: the first rows of every destination chunk
    (an exact sub-problem: same P, N, K and chunk structure)."""
    import numpy as np

    want = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "16") or 16), 16)
    import oracle
    oracle.set_threads(want)
    cores = oracle.max_threads()
    from computation_collective_amd import configs as cfgs
    from computation_collective_amd import inputs as gen

    c = cfgs.GEMM_RS_MLP
    Mc = c.M // c.P

    A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, c.in_dt, seed=0)

    def run(rows_per_chunk):
        sel = np.concatenate([np.arange(r * Mc, r * Mc + rows_per_chunk) for r in range(c.P)])
        As = np.ascontiguousarray(A[:, sel, :])
        Ms = c.P * rows_per_chunk
        t0 = time.perf_counter()
        oracle.gemm_rs(c.P, Ms, c.N, c.K, c.in_dt, c.slot_dt, c.out_dt, As, W, want_slots=False)
        dt = time.perf_counter() - t0
        return dt, 2.0 * c.P * Ms * c.N * c.K

    dt, fl = run(1)
    rows = max(1, min(Mc, int(target_s / max(dt, 1e-3))))
    dt, fl = run(rows)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{rows} rows of each of the {c.P} destination chunks ({c.P * rows} of {c.M} "
                      f"output rows) of gemm_rs P={c.P} {c.M}x{c.N}x{c.K} bf16, fp32 partials"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from computation_collective_amd import buffers as bf
    from computation_collective_amd import configs as cfgs
    from computation_collective_amd import hocf
    from computation_collective_amd import inputs as gen

    if not os.path.exists(hocf.LIB_PATH):
        from computation_collective_amd import build as hip_build
        hip_build.build()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    ops = [o for o in args.ops.split(",") if o]
    sdt = bf.F32 if args.slot_dtype == "f32" else bf.BF16
    runs = {}
    # a 1 GiB scratch read before a timed call (untimed: each call has its own events) leaves
    # none of the operator's data in the 256 MB Infinity Cache, only clean lines of the scratch
    # buffer (a scratch write would leave dirty lines, written back inside the timed call), and
    # the same cache state whatever ran before; used by the embedding bag and by both GEMV
    # variants (so that the fused and the unfused GEMV start alike)
    flush_buf = {}

    def mall_flush():
        if "t" not in flush_buf:
            flush_buf["t"] = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
            flush_buf["s"] = torch.empty((), dtype=torch.float32, device=dev)
        torch.sum(flush_buf["t"], dim=0, out=flush_buf["s"])

    if "gemm_rs" in ops:
        c = cfgs.GEMM_RS_MLP
        log(f"inputs {c.name}")
        A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, c.in_dt, seed=0)
        r = bf.GemmRS(c.P, c.M, c.N, c.K, c.in_dt, sdt, c.out_dt, c.tile_m, c.tile_n, A, W)
        del A, W
        flops = c.flops
        algo_bytes = (2 * (c.P * c.M * c.K + c.P * c.K * c.N)            # A, W read
                      + 2 * (4 if sdt == bf.F32 else 2) * c.P * c.M * c.N  # slots written + read
                      + 2 * c.M * c.N)                                     # out written
        runs["gemm_rs"] = dict(call=lambda r=r: r.run(stream), obj=r, work=flops, unit="TFLOP/s",
                               variant=f"slot_dtype={args.slot_dtype} tile={c.tile_m}x{c.tile_n}",
                               bound="mfma", peak=PEAK_BF16_TFLOPS, bytes=algo_bytes,
                               config=dict(workload=c.name, P=c.P, M=c.M, N=c.N, K=c.K,
                                           tile=[c.tile_m, c.tile_n], slot_dtype=args.slot_dtype))
    if "gemm_rs_tiny" in ops:
        c = cfgs.GEMM_RS_TINY
        log(f"inputs {c.name}")
        A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, c.in_dt, seed=0, dist_a=c.dist_a, dist_w=c.dist_w)
        rt = bf.GemmRS(c.P, c.M, c.N, c.K, c.in_dt, c.slot_dt, c.out_dt, c.tile_m, c.tile_n, A, W)
        algo_bytes = (4 * (c.P * c.M * c.K + c.P * c.K * c.N)      # A, W read
                      + 2 * 4 * c.P * c.M * c.N                    # slots written + read
                      + 4 * c.M * c.N)                             # out written
        runs["gemm_rs_tiny"] = dict(call=lambda r=rt: r.run(stream), obj=rt, work=c.flops, unit="TFLOP/s",
                                    variant=f"tile={c.tile_m}x{c.tile_n}", bound="mfma", peak=PEAK_F32_TFLOPS,
                                    bytes=algo_bytes,
                                    config=dict(workload=c.name, P=c.P, M=c.M, N=c.N, K=c.K,
                                                tile=[c.tile_m, c.tile_n], dtype="f32",
                                                peak_note="fp32 MFMA 157.3 TFLOP/s"))
    if "gemv_ar" in ops:
        c = cfgs.GEMV_AR_DECODE
        log(f"inputs {c.name}")
        x, W = gen.gemv_ar_inputs(c.P, c.Mb, c.N, c.K, seed=0)
        gtile = args.gemv_tile or c.tile_n
        g = bf.GemvAR(c.P, c.Mb, c.N, c.K, c.in_dt, c.slot_dt, c.out_dt, gtile, x, W)
        # 4 replicas of the weights (537 MB > the 256 MB Infinity Cache) rotate per call
        reps = [(g.x, g.W)] + [(g.x.clone(), g.W.clone()) for _ in range(3)]
        state = {"i": 0}

        def gemv_call(g=g, reps=reps, state=state):
            xr, Wr = reps[state["i"] % len(reps)]
            state["i"] += 1
            g.set_weights(xr, Wr)
            g.run(stream)

        algo_bytes = (2 * c.P * c.K * c.N + 2 * c.P * c.Mb * c.K          # W, x read
                      + 2 * 4 * c.P * c.Mb * c.N                          # partials written + read
                      + 2 * c.P * c.Mb * c.N)                             # P windows written
        runs["gemv_ar"] = dict(call=gemv_call, obj=g, work=algo_bytes, unit="GB/s", bound="hbm", pre=mall_flush,
                               variant=f"tile_n={gtile} weight_replicas=4",
                               peak=PEAK_HBM_GBS, bytes=algo_bytes, flops=c.flops,
                               config=dict(workload=c.name, P=c.P, Mb=c.Mb, N=c.N, K=c.K, tile_n=gtile,
                                           weight_replicas=4))
    if "ag_gemm" in ops:
        c = cfgs.AG_GEMM_COL
        log(f"inputs {c.name}")
        chunks, W, order = gen.ag_gemm_inputs(c.P, c.Mc, c.N, c.K, seed=0)
        a = bf.AgGemm(c.P, c.Mc, c.N, c.K, bf.BF16, c.tile_m, c.tile_n, chunks, W)

        ag_state = {}

        def ag_pre(a=a, order=order, st=ag_state):
            # the chunk flags, written in the seeded order on the kernel's own stream before the
            # kernel (stream write-values: the runtime runs each as a one-workgroup kernel);
            # outside the timed events: the kernel's span is timed
            st["sync"] = a.prerelease(order, stream=stream)

        def ag_call(a=a, st=ag_state):
            a.launch(st["sync"], stream)

        algo_bytes = 2 * (c.P * c.Mc * c.K + c.K * c.N + c.P * c.Mc * c.N)
        runs["ag_gemm"] = dict(call=ag_call, pre=ag_pre, obj=a, work=c.flops, unit="TFLOP/s", bound="mfma",
                               variant=f"tile={c.tile_m}x{c.tile_n} prereleased",
                               peak=PEAK_BF16_TFLOPS, bytes=algo_bytes,
                               config=dict(workload=c.name, P=c.P, Mc=c.Mc, N=c.N, K=c.K,
                                           tile=[c.tile_m, c.tile_n], release_order=[int(v) for v in order]))
    if "ag_gemm_paced" in ops:
        # context: the chunks arrive over time, as over xGMI (8 MB per chunk at ~153 GB/s per
        # link: one every ~55 us), the first (the local one) at the start; chunk data resident,
        # flags in host-coherent memory written by the host on a busy-wait clock after the launch
        c = cfgs.AG_GEMM_COL
        log(f"inputs {c.name} (paced arrival)")
        chunks, W, order = gen.ag_gemm_inputs(c.P, c.Mc, c.N, c.K, seed=0)
        ap_ = bf.AgGemm(c.P, c.Mc, c.N, c.K, bf.BF16, c.tile_m, c.tile_n, chunks, W, flags="host")
        gap_s = args.chunk_gap_us * 1e-6

        def ag_paced_call(a=ap_, order=order):
            sy = a.next_sync(spin_timeout_ns=2_000_000_000)
            hocf.check(a.call(sy, stream))
            t0 = time.perf_counter()
            for k, ch in enumerate(order):
                while time.perf_counter() - t0 < k * gap_s:
                    pass
                a.host_flags[int(ch)] = sy.epoch

        runs["ag_gemm_paced"] = dict(call=ag_paced_call, pre=torch.cuda.synchronize, obj=ap_, work=c.flops,
                                     unit="TFLOP/s", bound="mfma", peak=PEAK_BF16_TFLOPS,
                                     bytes=2 * (c.P * c.Mc * c.K + c.K * c.N + c.P * c.Mc * c.N),
                                     config=dict(workload=c.name + "_paced", P=c.P, Mc=c.Mc, N=c.N, K=c.K,
                                                 tile=[c.tile_m, c.tile_n], chunk_gap_us=args.chunk_gap_us,
                                                 arrival_span_us=(c.P - 1) * args.chunk_gap_us,
                                                 release_order=[int(v) for v in order]))
    # HOCCL's copy-engine communication on one GPU: the AllGather's seven remote 8 MB chunks
    # moved by hocf_dma_put (each chunk's bytes, then its flag) on a second stream, either on
    # the copy (SDMA) engines with no compute unit, or on the runtime's copy kernels
    put_ops = [o for o in ("ag_gemm_dma", "ag_gemm_cu_put", "dma_put", "cu_put", "gemm_rs_dma_put",
                           "gemm_rs_cu_put") if o in ops]
    if put_ops:
        # one small put on each engine first: a runtime without copy-engine support drops
        # these operators (logged) rather than the whole bench line
        probe = torch.zeros(2, 1 << 16, dtype=torch.int32, device=dev)
        for eng in (hocf.HOCF_ENGINE_DMA, hocf.HOCF_ENGINE_CU):
            st = hocf.hocf_dma_put([probe[0]], [probe[1]], [1 << 18], None, None, eng, torch.cuda.current_stream())
            if st != hocf.HOCF_OK:
                log(f"copy-engine puts skipped: engine {eng}: {hocf.last_error()}")
                put_ops = []
        torch.cuda.synchronize()
    if put_ops:
        c = cfgs.AG_GEMM_COL
        log(f"inputs {c.name} (copy-engine puts: {', '.join(put_ops)})")
        put_stream = torch.cuda.Stream(device=dev)
        chunks, W, order = gen.ag_gemm_inputs(c.P, c.Mc, c.N, c.K, seed=0)
        local = int(order[0])          # this rank's own chunk: in place, its put only signals
        chunk_bytes = 2 * c.Mc * c.K
        remote = [int(q) for q in order if int(q) != local]
        put_bytes = chunk_bytes * len(remote)
        engines = {"dma": hocf.HOCF_ENGINE_DMA, "cu": hocf.HOCF_ENGINE_CU}
        for name, eng in (("ag_gemm_dma", "dma"), ("ag_gemm_cu_put", "cu")):
            if name not in put_ops:
                continue
            ad = bf.AgGemm(c.P, c.Mc, c.N, c.K, bf.BF16, c.tile_m, c.tile_n, chunks, W)
            sends = [None if q == local else ad.A[q].clone() for q in range(c.P)]

            def ag_put_call(a=ad, sends=sends, engine=engines[eng]):
                a.put_delivered(sends, order, engine, put_stream, stream=stream,
                                spin_timeout_ns=2_000_000_000)

            runs[name] = dict(call=ag_put_call, obj=ad, work=c.flops, unit="TFLOP/s", bound="mfma",
                              peak=PEAK_BF16_TFLOPS, variant=f"tile={c.tile_m}x{c.tile_n} {eng} puts",
                              bytes=2 * (c.P * c.Mc * c.K + c.K * c.N + c.P * c.Mc * c.N) + 2 * put_bytes,
                              put_bytes=put_bytes,
                              config=dict(workload=f"{c.name}_{eng}_put", P=c.P, Mc=c.Mc, N=c.N, K=c.K,
                                          tile=[c.tile_m, c.tile_n], engine=eng, put_bytes=put_bytes,
                                          release_order=[int(v) for v in order]))
        # the same seven puts alone, and beside the GEMM+ReduceScatter kernel (which holds every CU)
        psrc = [torch.from_numpy(chunks[q].view(np.int16)).to(dev) for q in remote]
        pdst = torch.empty((len(remote), c.Mc * c.K), dtype=torch.int16, device=dev)

        def enqueue_puts(engine):
            put_stream.wait_stream(stream)
            # no signals: whatever consumes the bytes is ordered after the puts by the streams
            hocf.check(hocf.hocf_dma_put(psrc, [pdst[i] for i in range(len(remote))], [chunk_bytes] * len(remote),
                                         None, None, engine, put_stream))

        for name, eng in (("dma_put", "dma"), ("cu_put", "cu")):
            if name not in put_ops:
                continue

            def put_call(engine=engines[eng]):
                enqueue_puts(engine)
                stream.wait_stream(put_stream)

            runs[name] = dict(call=put_call, obj=None, work=2 * put_bytes, unit="GB/s", bound="hbm",
                              peak=PEAK_HBM_GBS, bytes=2 * put_bytes, put_bytes=put_bytes,
                              config=dict(workload=f"put_7x8MB_{eng}", engine=eng, puts=len(remote),
                                          put_bytes=put_bytes))
        gr = [o for o in ("gemm_rs_dma_put", "gemm_rs_cu_put") if o in put_ops]
        if gr:
            cg = cfgs.GEMM_RS_MLP
            if "gemm_rs" in runs:
                rg = runs["gemm_rs"]["obj"]
            else:
                A_, W_ = gen.gemm_rs_inputs(cg.P, cg.M, cg.N, cg.K, cg.in_dt, seed=0)
                rg = bf.GemmRS(cg.P, cg.M, cg.N, cg.K, cg.in_dt, sdt, cg.out_dt, cg.tile_m, cg.tile_n, A_, W_)
                del A_, W_
            for name in gr:
                eng = "dma" if name == "gemm_rs_dma_put" else "cu"

                marks = []

                def gemm_put_call(engine=engines[eng], r=rg, marks=marks):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    enqueue_puts(engine)       # first, so the puts do not wait for the GEMM
                    r.run(stream)
                    b.record(stream)           # the GEMM's own end, before the wait for the puts
                    marks.append((a, b))
                    stream.wait_stream(put_stream)

                runs[name] = dict(call=gemm_put_call, obj=rg, work=cg.flops, unit="TFLOP/s", bound="mfma",
                                  peak=PEAK_BF16_TFLOPS, bytes=0, put_bytes=put_bytes, marks=marks,
                                  variant=f"slot_dtype={args.slot_dtype} tile={cg.tile_m}x{cg.tile_n} {eng} puts",
                                  config=dict(workload=f"{cg.name}_with_{eng}_puts_7x8MB", engine=eng,
                                              put_bytes=put_bytes, slot_dtype=args.slot_dtype))
    if "embbag_a2a" in ops:
        c = cfgs.EMBBAG_DLRM
        log(f"inputs {c.name} (tables on the device)")
        tables = gen.embbag_tables_torch(c.T, c.R, c.D, seed=0, device=dev)
        idx = gen.zipf_indices(c.T, c.B, c.L, c.R, alpha=c.alpha, seed=0)
        e = bf.EmbbagA2A(c.T, c.R, c.D, c.B, c.L, c.P, c.tile_bags, tables, idx)
        logical = (4 * c.T * c.B * c.L * c.D          # every looked-up row (Zipf repeats included)
                   + 4 * c.T * c.B * c.L              # indices
                   + 4 * c.T * c.B * c.D)             # pooled rows written to the buckets
        uniq = sum(int(np.unique(idx[t]).size) for t in range(c.T))
        compulsory = (4 * uniq * c.D                  # every distinct row once
                      + 4 * c.T * c.B * c.L           # indices
                      + 4 * c.T * c.B * c.D)          # pooled rows written to the buckets
        del idx
        # the 1 GiB scratch read between calls (untimed: each call has its own events) keeps the
        # 256 MB Infinity Cache from carrying rows over from the previous call; reuse inside a
        # call (Zipf) is the workload's own locality
        runs["embbag_a2a"] = dict(call=lambda e=e: e.run(stream), obj=e, work=compulsory, unit="GB/s",
                                  pre=mall_flush, logical=logical,
                                  variant=f"tile_bags={c.tile_bags}",
                                  bound="hbm", peak=PEAK_HBM_GBS, bytes=compulsory,
                                  config=dict(workload=c.name, T=c.T, R=c.R, D=c.D, B=c.B, L=c.L, P=c.P,
                                              tile_bags=c.tile_bags, zipf_alpha=c.alpha, distinct_rows=uniq,
                                              bytes="compulsory: distinct rows once + indices + pooled rows"))
    if "gemm_ar" in ops:
        c = cfgs.GEMM_AR_MLP
        log(f"inputs {c.name}")
        A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, c.in_dt, seed=0)
        ar = bf.GemmAR(c.P, c.M, c.N, c.K, c.in_dt, sdt, c.out_dt, c.tile_m, c.tile_n, A, W)
        del A, W
        algo_bytes = (2 * (c.P * c.M * c.K + c.P * c.K * c.N)            # A, W read
                      + 2 * (4 if sdt == bf.F32 else 2) * c.P * c.M * c.N  # slots written + read
                      + 2 * c.P * c.M * c.N)                               # P full windows written
        runs["gemm_ar"] = dict(call=lambda r=ar: r.run(stream), obj=ar, work=c.flops, unit="TFLOP/s",
                               variant=f"slot_dtype={args.slot_dtype} tile={c.tile_m}x{c.tile_n}",
                               bound="mfma", peak=PEAK_BF16_TFLOPS, bytes=algo_bytes,
                               config=dict(workload=c.name, P=c.P, M=c.M, N=c.N, K=c.K,
                                           tile=[c.tile_m, c.tile_n], slot_dtype=args.slot_dtype))
    if "gemm_a2a" in ops:
        c = cfgs.GEMM_A2A_MOE
        log(f"inputs {c.name}")
        atm = args.a2a_tile_m or c.tile_m
        off, dest, slot, counts = gen.moe_routing(c.P, c.E, c.B, c.topk, atm, seed=0)
        X, W = gen.gemm_a2a_inputs(c.E, int(off[-1]), c.N, c.K, dest, seed=0)
        ga = bf.GemmA2A(c.P, c.E, c.N, c.K, bf.BF16, X, W, off, dest, slot, counts, c.cap, tile_m=atm)
        rows = int(counts.sum())
        del X, W
        flops = 2.0 * rows * c.N * c.K                    # the routed rows (padding rows excluded)
        algo_bytes = (2 * int(off[-1]) * c.K + 2 * c.E * c.K * c.N   # X, W read
                      + 8 * int(off[-1])                            # dest, slot
                      + 2 * rows * c.N)                             # result rows written
        runs["gemm_a2a"] = dict(call=lambda r=ga: r.run(stream), obj=ga, work=flops, unit="TFLOP/s",
                                variant=f"tile={atm}x{c.tile_n}", bound="mfma", peak=PEAK_BF16_TFLOPS,
                                bytes=algo_bytes,
                                config=dict(workload=c.name, P=c.P, E=c.E, B=c.B, topk=c.topk, N=c.N, K=c.K,
                                            cap=c.cap, rows=rows, padded_rows=int(off[-1]),
                                            tile=[atm, c.tile_n]))
    for a2g_op in ("a2a_gemm", "a2a_gemm_unfused"):
        if a2g_op not in ops:
            continue
        # the MoE dispatch: routing (counts, prefix sums, row placement) and row delivery on the
        # device, then the expert GEMM; the unfused form delivers every row before any tile starts
        c = cfgs.A2A_GEMM_MOE
        log(f"inputs {c.name}" + (" (unfused)" if a2g_op.endswith("unfused") else ""))
        experts = gen.moe_choices(c.P, c.E, c.B, c.topk, seed=0)
        X, W = gen.a2a_gemm_inputs(c.P, c.B, c.K, c.E, c.N, seed=0)
        dg = bf.A2aGemm(c.P, c.E, 0, c.B, c.topk, c.N, c.K, bf.BF16, X, experts, W, c.cap, tile_m=c.tile_m,
                        unfused=a2g_op.endswith("unfused"))
        del X, W
        n_e = np.bincount(experts[experts < c.E].ravel(), minlength=c.E)
        rows = int(n_e.sum())
        padded = int(sum(-(-int(n) // c.tile_m) * c.tile_m for n in n_e))
        flops = 2.0 * rows * c.N * c.K                        # the routed rows (padding rows excluded)
        algo_bytes = (4 * c.P * c.B * c.topk                  # router choices
                      + 2 * rows * c.K                        # token rows read
                      + 2 * 2 * padded * c.K                  # received rows written, then read by the GEMM
                      + 2 * c.E * c.K * c.N                   # W read
                      + 2 * padded * c.N)                     # Y written
        runs[a2g_op] = dict(call=lambda r=dg: r.run(stream), obj=dg, work=flops, unit="TFLOP/s", bound="mfma",
                            variant=f"tile={c.tile_m}x{c.tile_n}", peak=PEAK_BF16_TFLOPS, bytes=algo_bytes,
                            config=dict(workload=c.name + ("_unfused" if a2g_op.endswith("unfused") else ""),
                                        P=c.P, E=c.E, B=c.B, topk=c.topk, N=c.N, K=c.K, cap=c.cap, rows=rows,
                                        padded_rows=padded, tile=[c.tile_m, c.tile_n]))
    for o in [o for o in ops if o.startswith("gemm_rs_decomp")]:
        # Compass's InterDecom on one GPU: the gemm_rs workload in d column pieces, each piece's
        # GEMM on the step's stream (leaving F CUs free), its fold on a second stream:
        # gemm_rs_decomp<d>_f<F> (e.g. gemm_rs_decomp4_f32)
        d_, f_ = o[len("gemm_rs_decomp"):].split("_f")
        c = cfgs.GEMM_RS_MLP
        log(f"inputs {c.name} (decomposed, {d_} pieces, {f_} CUs for the folds)")
        A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, c.in_dt, seed=0)
        dr = bf.GemmRS(c.P, c.M, c.N, c.K, c.in_dt, sdt, c.out_dt, c.tile_m, c.tile_n, A, W, pieces=int(d_),
                       fold_cus=int(f_))
        del A, W
        runs[o] = dict(call=lambda r=dr: r.run(stream), obj=dr, work=c.flops, unit="TFLOP/s", bound="mfma",
                       variant=f"slot_dtype={args.slot_dtype} tile={c.tile_m}x{c.tile_n} pieces={d_} fold_cus={f_}",
                       peak=PEAK_BF16_TFLOPS,
                       bytes=(2 * (c.P * c.M * c.K + c.P * c.K * c.N)
                              + 2 * (4 if sdt == bf.F32 else 2) * c.P * c.M * c.N + 2 * c.M * c.N),
                       config=dict(workload=c.name + f"_decomposed_d{d_}_f{f_}", P=c.P, M=c.M, N=c.N, K=c.K,
                                   tile=[c.tile_m, c.tile_n], pieces=int(d_), fold_cus=int(f_),
                                   slot_dtype=args.slot_dtype))
    if "gemm_rs_unfused" in ops:
        # the baseline of the fused operator: the same GEMM, then a separate fold kernel
        c = cfgs.GEMM_RS_MLP
        log(f"inputs {c.name} (unfused)")
        A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, c.in_dt, seed=0)
        u = bf.GemmRS(c.P, c.M, c.N, c.K, c.in_dt, sdt, c.out_dt, c.tile_m, c.tile_n, A, W, unfused=True)
        del A, W
        algo_bytes = (2 * (c.P * c.M * c.K + c.P * c.K * c.N)
                      + 2 * (4 if sdt == bf.F32 else 2) * c.P * c.M * c.N + 2 * c.M * c.N)
        runs["gemm_rs_unfused"] = dict(call=lambda r=u: r.run(stream), obj=u, work=c.flops, unit="TFLOP/s",
                                       variant=f"slot_dtype={args.slot_dtype} tile={c.tile_m}x{c.tile_n}",
                                       bound="mfma", peak=PEAK_BF16_TFLOPS, bytes=algo_bytes,
                                       config=dict(workload=c.name + "_unfused", P=c.P, M=c.M, N=c.N, K=c.K,
                                                   tile=[c.tile_m, c.tile_n], slot_dtype=args.slot_dtype,
                                                   kernels="GEMM (tiles published), then the fold"))
    if "gemv_ar_unfused" in ops:
        # the baseline of the fused GEMV + AllReduce: the GEMV, then a separate fold kernel
        c = cfgs.GEMV_AR_DECODE
        log(f"inputs {c.name} (unfused)")
        x, W = gen.gemv_ar_inputs(c.P, c.Mb, c.N, c.K, seed=0)
        gtile = args.gemv_tile or c.tile_n
        gu = bf.GemvAR(c.P, c.Mb, c.N, c.K, c.in_dt, c.slot_dt, c.out_dt, gtile, x, W, unfused=True)
        ureps = [(gu.x, gu.W)] + [(gu.x.clone(), gu.W.clone()) for _ in range(3)]
        ustate = {"i": 0}

        def gemv_u_call(g=gu, reps=ureps, state=ustate):
            xr, Wr = reps[state["i"] % len(reps)]
            state["i"] += 1
            g.set_weights(xr, Wr)
            g.run(stream)

        algo_bytes = (2 * c.P * c.K * c.N + 2 * c.P * c.Mb * c.K + 2 * 4 * c.P * c.Mb * c.N
                      + 2 * c.P * c.Mb * c.N)
        runs["gemv_ar_unfused"] = dict(call=gemv_u_call, obj=gu, work=algo_bytes, unit="GB/s", bound="hbm",
                                       pre=mall_flush,
                                       variant=f"tile_n={gtile} weight_replicas=4",
                                       peak=PEAK_HBM_GBS, bytes=algo_bytes,
                                       config=dict(workload=c.name + "_unfused", P=c.P, Mb=c.Mb, N=c.N, K=c.K,
                                                   tile_n=gtile, weight_replicas=4,
                                                   kernels="GEMV (partials published), then the fold"))
    if "hipblaslt_bmm" in ops:
        # context, not a fused operator: the vendor library (torch.bmm -> hipBLASLt) on the same
        # eight shard GEMMs as gemm_rs, bf16 in, bf16 out, with no collective at all; both
        # operands contiguous (a transposed view as the right operand is avoided)
        c = cfgs.GEMM_RS_MLP
        log(f"inputs {c.name} (hipBLASLt context)")
        A, W = gen.gemm_rs_inputs(c.P, c.M, c.N, c.K, c.in_dt, seed=0)
        At = bf.to_device(A, dev).view(torch.bfloat16).contiguous()
        Wt = bf.to_device(W, dev).view(torch.bfloat16).contiguous()
        Ct = torch.empty((c.P, c.M, c.N), dtype=torch.bfloat16, device=dev)
        del A, W
        runs["hipblaslt_bmm"] = dict(call=lambda a=At, w=Wt, o=Ct: torch.bmm(a, w, out=o), obj=None, work=c.flops,
                                     unit="TFLOP/s", bound="mfma", peak=PEAK_BF16_TFLOPS,
                                     bytes=2 * (c.P * c.M * c.K + c.P * c.K * c.N + c.P * c.M * c.N),
                                     config=dict(workload=c.name + "_hipblaslt_bmm", P=c.P, M=c.M, N=c.N, K=c.K,
                                                 note="torch.bmm on the 8 shard GEMMs, no collective (context)"))
        # the same with fp32 output (the partials gemm_rs carries), where this torch build has it
        try:
            Cf = torch.bmm(At, Wt, out_dtype=torch.float32)
            torch.cuda.synchronize()
            runs["hipblaslt_bmm_f32out"] = dict(
                call=lambda a=At, w=Wt: torch.bmm(a, w, out_dtype=torch.float32), obj=None, work=c.flops,
                unit="TFLOP/s", bound="mfma", peak=PEAK_BF16_TFLOPS,
                bytes=2 * (c.P * c.M * c.K + c.P * c.K * c.N) + 4 * c.P * c.M * c.N,
                config=dict(workload=c.name + "_hipblaslt_bmm_f32out", P=c.P, M=c.M, N=c.N, K=c.K,
                            note="torch.bmm, fp32 output, on the 8 shard GEMMs, no collective (context)"))
            del Cf
        except (RuntimeError, TypeError, NotImplementedError) as ex:
            log(f"hipBLASLt fp32-output context skipped: {type(ex).__name__}")
    if "embbag_uniform" in ops:
        # control: the same shapes with uniform indices (no reuse), so logical ~ DRAM bytes
        c = cfgs.EMBBAG_DLRM
        if "embbag_a2a" not in ops:
            tables = gen.embbag_tables_torch(c.T, c.R, c.D, seed=0, device=dev)
        uidx = gen.uniform_indices(c.T, c.B, c.L, c.R, seed=1)
        eu = bf.EmbbagA2A(c.T, c.R, c.D, c.B, c.L, c.P, c.tile_bags, tables, uidx)
        logical_u = 4 * c.T * c.B * c.L * c.D + 4 * c.T * c.B * c.L + 4 * c.T * c.B * c.D
        uniq_u = sum(int(np.unique(uidx[t]).size) for t in range(c.T))
        algo_bytes = 4 * uniq_u * c.D + 4 * c.T * c.B * c.L + 4 * c.T * c.B * c.D
        runs["embbag_uniform"] = dict(call=lambda e=eu: e.run(stream), obj=eu, work=algo_bytes, unit="GB/s",
                                      pre=mall_flush, variant="uniform indices", logical=logical_u,
                                      bound="hbm", peak=PEAK_HBM_GBS, bytes=algo_bytes,
                                      config=dict(workload=c.name + "_uniform_indices", T=c.T, R=c.R, D=c.D,
                                                  B=c.B, L=c.L, P=c.P, tile_bags=c.tile_bags))
    if "copy" in ops:
        # a plain elementwise pass over 1 GiB (read 1 GiB, write 1 GiB; a negating copy, so its
        # kernel is told apart from the runtime's own copies): the calibration of the HBM counters
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        runs["copy"] = dict(call=lambda src=src, dst=dst: torch.neg(src, out=dst), obj=None, work=2 * nbytes,
                            unit="GB/s", bound="hbm", peak=PEAK_HBM_GBS, bytes=2 * nbytes,
                            config=dict(workload="device copy 1 GiB (counter calibration)"))
    torch.cuda.synchronize()

    # timed in the order --ops lists them (operators added under another name last)
    names = [o for o in ops if o in runs] + [n for n in runs if n not in ops]
    ev = {n: [] for n in names}

    # every other step swaps the two members of each fused / unfused pair, so each follows
    # the other half of the time and the operator before the pair the other half (an
    # operator that comes right after a large GEMM measures slower than in isolation)
    nstep = {"i": 0}
    swapped = list(names)
    for i in range(len(swapped) - 1):
        if swapped[i + 1] == swapped[i] + "_unfused":
            swapped[i], swapped[i + 1] = swapped[i + 1], swapped[i]

    def step(record):
        order = names if nstep["i"] % 2 == 0 else swapped
        nstep["i"] += 1
        for n in order:
            if "pre" in runs[n]:
                runs[n]["pre"]()
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                runs[n]["call"]()
                e1.record(stream)
                ev[n].append((e0, e1))
            else:
                runs[n]["call"]()

    log(f"warmup {args.warmup}")
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step(False)
    torch.cuda.synchronize()
    log(f"timed {args.steps} steps")
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    for n in names:
        if runs[n]["obj"] is None:
            continue
        st = runs[n]["obj"].status_value()
        if st != 0:
            raise SystemExit(f"{n}: device status {st} ({hocf.status_string(st)})")

    from computation_collective_amd import profsum
    out_ops = {}
    for n in names:
        ms = [a.elapsed_time(b) for a, b in ev[n]]
        avg = sum(ms) / len(ms)
        R = runs[n]
        scale = 1e12 if R["unit"] == "TFLOP/s" else 1e9
        v = R["work"] / (avg * 1e-3) / scale          # per launch, over the average launch duration
        tb = profsum.traffic(n, R.get("variant"))      # scaled HBM bytes per launch, if current
        srt = sorted(ms)
        out_ops[n] = {
            "value": round(v, 2), "unit": R["unit"], "ms_avg": round(avg, 4), "ms_median": round(median(ms), 4),
            "ms_p10": round(srt[int(0.1 * (len(srt) - 1))], 4), "ms_p90": round(srt[int(0.9 * (len(srt) - 1))], 4),
            "ms_min": round(min(ms), 4), "ms_max": round(max(ms), 4),
            "roofline": {"bound": R["bound"], "achieved": round(v, 2), "peak": R["peak"],
                         "unit": R["unit"] if R["bound"] == "mfma" else "GB/s",
                         "frac": round(v / R["peak"], 4), "traffic": None if tb is None else int(tb)},
            "algo_bytes": R["bytes"],
            # bytes between the L2s and the memory fabric (the FETCH_SIZE and WRITE_SIZE counters,
            # calibrated on a copy of known size): the fabric side of the L2s, where the 256 MB
            # Infinity Cache may still serve a part; null until a profile of the current sources exists
            "l2_fabric": None if tb is None else {
                "bytes": int(tb), "gbps": round(tb / (avg * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(tb / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "config": R["config"],
        }
        if "logical" in R:
            out_ops[n]["logical_gbps"] = round(R["logical"] / (avg * 1e-3) / 1e9, 1)
        if "put_bytes" in R:
            # the puts' own rate: bytes delivered over the call's span
            out_ops[n]["put_gbps"] = round(R["put_bytes"] / (avg * 1e-3) / 1e9, 1)
        if "marks" in R:
            # the kernel's own span (from before the puts to its end), apart from the wait for the puts
            km = [a.elapsed_time(b) for a, b in R["marks"][-len(ms):]]
            out_ops[n]["kernel_ms_avg"] = round(sum(km) / len(km), 4)
            log(f"{n}: kernel {sum(km) / len(km):.4f} ms of the {avg:.4f} ms span")
        if n == "ag_gemm_paced":
            # how long the kernel runs on after the last chunk has arrived
            out_ops[n]["after_last_arrival_us"] = round(avg * 1e3 - R["config"]["arrival_span_us"], 1)
        log(f"{n}: {v:.1f} {R['unit']} ({avg:.4f} ms average, {100 * v / R['peak']:.1f}% of peak)")

    head = "gemm_rs" if "gemm_rs" in out_ops else names[0]
    res = {
        "metric": METRIC,
        "value": out_ops[head]["value"],
        "unit": out_ops[head]["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": out_ops[head]["config"]["workload"],
                   "step": "one call each of " + ", ".join(names),
                   "slot_dtype": args.slot_dtype},
        "roofline": out_ops[head]["roofline"],
        "ops": out_ops,
    }
    # fused against unfused (the computation, then the collective) on the same GPU
    fusion = {}
    for op in ("gemm_rs", "gemv_ar", "a2a_gemm"):
        if op in out_ops and op + "_unfused" in out_ops:
            f, u = out_ops[op]["ms_avg"], out_ops[op + "_unfused"]["ms_avg"]
            fusion[op] = {"fused_ms": f, "unfused_ms": u, "time_saved": round(1.0 - f / u, 4)}
            log(f"fusion: {op} fused {f:.4f} ms, unfused {u:.4f} ms ({100 * (1 - f / u):.1f}% less time)")
    # Compass's InterDecom (column pieces pipelined on two streams) against the same two
    decomp = {o: out_ops[o]["ms_avg"] for o in out_ops if o.startswith("gemm_rs_decomp")}
    if decomp and "gemm_rs" in fusion:
        fusion["gemm_rs"]["decomposed_ms"] = decomp
        for o, v in decomp.items():
            log(f"interdecom: {o} {v:.4f} ms (fused {fusion['gemm_rs']['fused_ms']:.4f}, "
                f"unfused {fusion['gemm_rs']['unfused_ms']:.4f})")
    if fusion:
        res["fusion"] = fusion
    if not args.no_cpu_baseline and "gemm_rs" in out_ops:
        log("cpu baseline (oracle on a bounded sample)")
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
