"""The rocprofv3 summaries behind profiles/ (comm_overlap_amd/profile_summary.py), on small result
databases written here with hand-computed answers: the trace form of the hidden copy time (copy
intervals covered by kernel intervals), HBM bytes scaled by a calibration copy, and the counter
ratios (clock, MFMA busy, waits, L1 -> L2 request latency and requests in flight)."""
import sqlite3

import pytest

from comm_overlap_amd import profile_summary as PS


def _db(path, kernels=(), copies=(), pmc=()):
    c = sqlite3.connect(path)
    c.execute("create table kernels (name text, grid_x int, start int, end int, dispatch_id int)")
    c.execute("create table memory_copies (name text, start int, end int, size int)")
    c.execute("create table pmc_events (name text, dispatch_id int, counter_name text, counter_value real)")
    c.execute("create table rocpd_kernel_dispatch (dispatch_id int, grid_size_x int)")
    for d, (name, grid, s, e) in enumerate(kernels):
        c.execute("insert into kernels values (?, ?, ?, ?, ?)", (name, grid, s, e, d))
        c.execute("insert into rocpd_kernel_dispatch values (?, ?)", (d, grid))
    c.executemany("insert into memory_copies values (?, ?, ?, ?)", copies)
    c.executemany("insert into pmc_events values (?, ?, ?, ?)", pmc)
    c.commit()
    c.close()
    return str(path)


def test_trace_overlap_of_copies_by_kernels(tmp_path, capsys):
    ms = 1_000_000  # ns
    db = _db(tmp_path / "t.db",
             kernels=[("gemm_kernel<A>", 65536, 1 * ms, 3 * ms), ("fence_kernel", 64, 3 * ms, 4 * ms),
                      ("gemm_kernel<A>", 65536, 4 * ms, 5 * ms)],
             copies=[("MEMORY_COPY_DEVICE_TO_DEVICE", 0, 2 * ms, 1 << 20),
                     ("MEMORY_COPY_DEVICE_TO_DEVICE", int(2.5 * ms), int(4.5 * ms), 1 << 20),
                     ("MEMORY_COPY_HOST_TO_DEVICE", 0, 10 * ms, 1 << 20)])
    assert PS.main(["trace", db]) == 0
    out = capsys.readouterr().out
    # the fence kernel does not match: covered 1 ms of the first copy, 0.5 + 0.5 ms of the second
    assert "overlapped by 'gemm_kernel' kernels: 50.0% of 4.000 ms" in out
    # two dispatches of 2000 and 1000 us
    line = next(l for l in out.splitlines() if l.strip().startswith("2 ") and "gemm_kernel<A>" in l)
    assert line.split()[:5] == ["2", "1500.00", "1000.00", "2000.00", "3.000"]


def test_traffic_scaled_by_the_calibration_copy(tmp_path, capsys):
    pmc_f = [("MulFunctor", 3, "FETCH_SIZE", 65536.0), ("MulFunctor", 3, "FETCH_SIZE", 65536.0),
             ("gemm_kernel<A>", 0, "FETCH_SIZE", 1000.0), ("gemm_kernel<A>", 1, "FETCH_SIZE", 3000.0),
             ("gemm_kernel<A>", 2, "FETCH_SIZE", 99999.0)]
    pmc_w = [("MulFunctor", 3, "WRITE_SIZE", 262144.0),
             ("gemm_kernel<A>", 0, "WRITE_SIZE", 400.0), ("gemm_kernel<A>", 1, "WRITE_SIZE", 600.0),
             ("gemm_kernel<A>", 2, "WRITE_SIZE", 99999.0)]
    kernels = [("gemm_kernel<A>", 65536, 0, 10), ("gemm_kernel<A>", 65536, 10, 20),
               ("gemm_kernel<A>", 1024, 20, 30), ("MulFunctor", 4096, 30, 40)]
    f = _db(tmp_path / "f.db", kernels=kernels, pmc=pmc_f)
    w = _db(tmp_path / "w.db", kernels=kernels, pmc=pmc_w)
    assert PS.main(["traffic", f, w, "--kernel", "gemm_kernel<A>", "--grid", "65536", "--calib-kernel",
                    "MulFunctor", "--calib-bytes", str(256 << 20)]) == 0
    out = capsys.readouterr().out
    # FETCH reads 131072 KiB for 256 MiB (scale 2), WRITE 262144 KiB (scale 1); the 1024-wide
    # dispatch is left out: 2000 KiB x 1024 x 2 + 500 KiB x 1024 x 1
    assert "scale 2.0000 (fetch), 1.0000 (write)" in out
    assert "2 fetch / 2 write dispatches" in out
    assert out.strip().splitlines()[-1] == f"traffic_bytes_per_launch: {2000 * 1024 * 2 + 500 * 1024}"


def test_counter_ratios(tmp_path, capsys):
    us = 1000  # ns
    cyc = 220_000  # per XCD over 100 us: 2.2 GHz
    pmc = []
    for d in (0, 1):
        pmc += [("gemm_kernel<A>", d, "GRBM_GUI_ACTIVE", 8.0 * cyc),
                ("gemm_kernel<A>", d, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * 1024),
                ("gemm_kernel<A>", d, "SQ_WAVE_CYCLES", 1e6), ("gemm_kernel<A>", d, "SQ_WAIT_ANY", 1e5),
                ("gemm_kernel<A>", d, "SQ_LDS_IDX_ACTIVE", 1e4), ("gemm_kernel<A>", d, "SQ_LDS_BANK_CONFLICT", 0.0)]
    db = _db(tmp_path / "c.db", kernels=[("gemm_kernel<A>", 65536, 0, 100 * us),
                                         ("gemm_kernel<A>", 65536, 200 * us, 300 * us)], pmc=pmc)
    assert PS.main(["counters", db]) == 0
    out = capsys.readouterr().out
    assert "2 dispatches, 100.0 us, clk 2.20 GHz, mfma_busy 50.0%, WAIT_ANY 10.0%, ldsconf 0.0%" in out


def test_request_latency_and_requests_in_flight(tmp_path, capsys):
    cyc = 1e6  # per XCD
    cus = 256
    passes = [
        {"SQ_LDS_DATA_FIFO_FULL": 0.0, "SQ_WAIT_INST_LDS": 5e4, "SQ_WAVE_CYCLES": 1e6},
        {"TD_TD_BUSY": 0.8 * cyc * cus, "TD_TC_STALL": 0.4 * cyc * cus, "TA_TA_BUSY": 0.57 * cyc * cus},
        {"TCP_PENDING_STALL_CYCLES": 0.44 * cyc * cus},
        {"TCP_TCC_READ_REQ": 1e6, "TCP_TCC_READ_REQ_LATENCY": 4e8, "TCC_HIT": 8e5, "TCC_MISS": 2e5,
         "TCC_EA0_RDREQ": 2e5, "TCC_EA0_RDREQ_LEVEL": 1.5e8},
    ]
    dbs = []
    for i, counters in enumerate(passes):
        # each counter split over two instances, as per-instance rows are summed
        pmc = [("gemm_kernel<A>", 0, "GRBM_GUI_ACTIVE", 8 * cyc)]
        for k, v in counters.items():
            pmc += [("gemm_kernel<A>", 0, k, v / 2), ("gemm_kernel<A>", 0, k, v / 2)]
        dbs.append(_db(tmp_path / f"p{i}.db", kernels=[("gemm_kernel<A>", 65536, 0, 500_000)], pmc=pmc))
    assert PS.main(["requests", *dbs]) == 0
    out = capsys.readouterr().out
    assert "duration under counters 500 us, clock 2.00 GHz" in out
    assert "L2 hit rate 0.800" in out
    assert "average TCP -> L2 read latency 400 cycles, average L2 miss latency 750 cycles" in out
    # 4e8 cycles of request latency over 1e6 cycles x 256 CUs
    assert f"reads in flight per CU {4e8 / (cyc * cus):.1f}" in out
    assert "TCP stalled on pending misses 0.44" in out
    assert "TD busy 0.80, stalled on the L1 0.40, TA busy 0.57" in out
    assert "waves waiting on LDS 0.05" in out


def test_instructions_per_mfma(tmp_path, capsys):
    pmc = []
    for d, scale in ((0, 1.0), (1, 1.0), (2, 3.0)):  # the median dispatch is one of the first two
        pmc += [("attn_fwd_kernel2", d, "SQ_INSTS_MFMA", 1000.0 * scale / 2), ("attn_fwd_kernel2", d, "SQ_INSTS_MFMA", 1000.0 * scale / 2),
                ("attn_fwd_kernel2", d, "SQ_INSTS_VALU", 3300.0 * scale), ("attn_fwd_kernel2", d, "SQ_INSTS_LDS", 700.0 * scale),
                ("attn_fwd_kernel2", d, "SQ_INSTS_VALU_TRANS_F32", 480.0 * scale)]
    pmc += [("attn_bwd_pre_kernel", 3, "SQ_INSTS_MFMA", 0.0), ("attn_bwd_pre_kernel", 3, "SQ_INSTS_VALU", 50.0),
            ("gemm_kernel<A>", 4, "SQ_INSTS_MFMA", 10.0)]
    db = _db(tmp_path / "i.db", pmc=pmc)
    assert PS.main(["insts", db]) == 0
    out = capsys.readouterr().out
    assert "attn_fwd_kernel2: 3 dispatches, per MFMA instruction: VALU 3.30, LDS 0.70, transcendental 0.48" in out
    assert "attn_bwd_pre_kernel: 1 dispatches, no MFMA instructions" in out
    assert "gemm_kernel" not in out


def test_missing_kernel_is_an_error(tmp_path):
    db = _db(tmp_path / "e.db", kernels=[("other", 64, 0, 10)],
             pmc=[("other", 0, "GRBM_GUI_ACTIVE", 8.0)])
    with pytest.raises(SystemExit):
        PS.main(["requests", db, db, db, db])
