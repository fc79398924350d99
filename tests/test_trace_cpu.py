"""Host logic of the trace summary (computation_collective_amd.trace) on
hand-built records: the overlap of folds with other workgroups' mainloops,
the phase split and the ready-to-folded latency (CPU only)."""

import numpy as np

from computation_collective_amd import trace as tr


def _rec(wg, it, ts, item, band, bits):
    return wg, it, ts, item, band, bits


def _records(rows):
    raw = np.zeros((tr.TRACE_WGS, tr.TRACE_ITERS, tr.REC_WORDS), dtype=np.uint64)
    for wg, it, ts, item, band, bits in rows:
        raw[wg, it, :6] = ts
        raw[wg, it, 6] = np.int64(item).view(np.uint64)
        raw[wg, it, 7] = (np.uint64(bits) << np.uint64(32)) | np.uint64(band & 0xFFFFFFFF)
    return raw.reshape(-1)


def _field(lines, key):
    for l in lines:
        if l.startswith(key):
            return dict(kv.split("=", 1) for kv in l.split() if "=" in kv)
    raise AssertionError(key)


def test_fold_during_another_workgroups_mainloop():
    # clock 100 MHz: 100 ticks = 1 us.  P = 2 shards, one output tile (1 x 1 tiles), 2 bands.
    # items: p * (tpc * P) + r * tpc + tile, so output tile 0 (chunk 0) gets items 0 (p 0) and 2 (p 1)
    # wg 0: tile item 0 mainloop 10..50 us; tile item 2 60..100 us, the last producer of output tile 0
    # wg 1: band 0 alone 102..110 us (wg 0 idle: no overlap); band 1 inside its own mainloop 20..58 us
    #       while wg 0 computes 20..50 (overlap 30 of 38 us)
    T = lambda *us: [int(1000 + 100 * u) for u in us]
    rows = [
        _rec(0, 0, T(0, 1, 10, 50, 55, 56), 0, -1, 0),
        _rec(0, 1, T(56, 57, 60, 100, 104, 105), 2, -1, tr.BIT_COMPLETED),
        _rec(1, 0, T(18, 19, 20, 58, 59, 60), 1, 1, tr.BIT_IN_LOOP),
        _rec(1, 1, T(101, 102, 110, 110, 110, 111), -1, 0, tr.BIT_ALONE),
    ]
    d = tr.parse(_records(rows), tr.TRACE_WGS)
    assert len(d["item"]) == 4
    lines = tr.summarize(d, 100_000, P=2, mtiles=1, ntiles=1, pieces=2)
    ov = _field(lines, "overlap")
    assert abs(float(ov["fold_time_us"]) - 46.0) < 0.6            # 38 in the loop + 8 alone
    assert abs(float(ov["share_with_one_or_more_other"]) - 30.0 / 46.0) < 0.02
    f = _field(lines, "folds")
    assert f["in_mainloop"] == "1" and f["alone"] == "1" and f["alone_without_tile"] == "1"
    lat = _field(lines, "ready_to_folded_us")
    assert lat["output_tiles_completed"] == "1"
    assert abs(float(lat["max"]) - 5.0) < 0.01                     # ready at 105, alone band done at 110
    ph = _field(lines, "phase_us")
    assert ph["mainloop_with_band"].startswith("38.00")


def test_output_tile_matches_the_kernels_item_order():
    # item = p * (tpc * P) + r * tpc + (column tile * mtiles + row tile)
    P, mtiles, ntiles = 3, 2, 4
    tpc = mtiles * ntiles
    for p in range(P):
        for r in range(P):
            for nt in range(ntiles):
                for mt in range(mtiles):
                    item = p * tpc * P + r * tpc + nt * mtiles + mt
                    assert tr.output_tile(item, P, mtiles, ntiles) == r * tpc + mt * ntiles + nt


def test_store_contention_counts_the_same_xcds_storers():
    # workgroups are dispatched round-robin over 8 XCDs: 0, 8 and 16 share XCD 0, 1 is on XCD 1.
    # wg 0 and wg 8 store 10..14 us together; wg 16 stores 30..32 us alone on its XCD;
    # wg 1 stores 10..12 us on another XCD (not counted against XCD 0)
    T = lambda *us: [int(1000 + 100 * u) for u in us]
    rows = [
        _rec(0, 0, T(0, 1, 2, 10, 14, 15), 0, 0, tr.BIT_IN_LOOP),
        _rec(8, 0, T(0, 1, 2, 10, 14, 15), 1, -1, 0),
        _rec(16, 0, T(20, 21, 22, 30, 32, 33), 2, -1, 0),
        _rec(1, 0, T(0, 1, 2, 10, 12, 13), 3, -1, 0),
    ]
    d = tr.parse(_records(rows), tr.TRACE_WGS)
    lines = tr.summarize(d, 100_000, P=2, mtiles=1, ntiles=2, pieces=2)
    line = next(l for l in lines if l.startswith("store_contention"))
    f = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
    assert abs(float(f["same_xcd_others_storing_mean"]) - 0.5) < 1e-9    # (1 + 1 + 0 + 0) / 4
    # all four below 8 others: store times 4, 4, 2, 2 us
    assert line.endswith("0-7:3.00,4")
