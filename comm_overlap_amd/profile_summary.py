"""Summaries of rocprofv3 runs of the sliced layer shard (reads the rocprofv3 SQLite output).

    python -m comm_overlap_amd.profile_summary trace RESULTS.db [--match gemm_kernel]
        per-kernel dispatch statistics, DMA-engine copies, and the share of copy time that
        overlaps kernels matching --match (the trace form of the hidden-copy fraction)
    python -m comm_overlap_amd.profile_summary traffic FETCH.db WRITE.db --kernel NAME
                                               --calib-kernel NAME --calib-bytes N
        HBM bytes per dispatch of NAME from a FETCH_SIZE pass and a WRITE_SIZE pass, each scaled
        by what the same counter reads for a calibration copy kernel that moves N bytes each way
        (--grid G: only NAME's dispatches with grid_size_x G, i.e. one product's shape)
    python -m comm_overlap_amd.profile_summary counters RESULTS.db [--match gemm_kernel]
        per kernel (medians over its dispatches) from a pass with GRBM_GUI_ACTIVE,
        SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, SQ_WAVE_CYCLES, SQ_WAIT_ANY:
        GRBM_GUI_ACTIVE reads the sum over the 8 XCDs, so one XCD's busy cycles are a eighth of it:
        clock = busy cycles / duration, MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (busy cycles x 1024
        SIMDs), wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES, LDS conflicts = SQ_LDS_BANK_CONFLICT /
        SQ_LDS_IDX_ACTIVE
    python -m comm_overlap_amd.profile_summary insts RESULTS.db [--match attn]
        per kernel (medians over its dispatches) from a pass with SQ_INSTS_VALU, SQ_INSTS_MFMA,
        SQ_INSTS_LDS and SQ_INSTS_VALU_TRANS_F32: the vector ALU, LDS and transcendental
        instructions issued per MFMA instruction
    python -m comm_overlap_amd.profile_summary requests P1.db P2.db P3.db P4.db [--match gemm_kernel]
        L1 -> L2 read requests of one kernel from four passes (SQ wave and LDS counters; TA/TD;
        TCP stalls; TCP -> L2 requests and L2 hits, misses and miss latency), each counter summed
        over its instances and taken as the median over the kernel's dispatches: hit rate, average
        request and miss latencies (latency sums / request counts), requests in flight per CU
        (request latency sum / (cycles x 256 CUs)) and the per-CU shares of cycles; cycles are
        GRBM_GUI_ACTIVE / 8 of the same pass
"""
from __future__ import annotations

import argparse
import collections
import sqlite3
import sys


def _kernels(db):
    c = sqlite3.connect(db)
    return list(c.execute("select name, start, end from kernels order by start"))


def _kernels_grid(db):
    c = sqlite3.connect(db)
    return list(c.execute("select name, grid_x, start, end from kernels order by start"))


def _copies(db):
    c = sqlite3.connect(db)
    try:
        return list(c.execute("select name, start, end, size from memory_copies order by start"))
    except sqlite3.OperationalError:
        return []


def _union(iv):
    out = []
    for s, e in sorted(iv):
        if out and s <= out[-1][1]:
            out[-1][1] = max(out[-1][1], e)
        else:
            out.append([s, e])
    return out


def trace(db, match):
    ks = _kernels(db)
    stats = collections.OrderedDict()
    for name, s, e in ks:
        d = stats.setdefault(name, [])
        d.append((e - s) / 1e3)
    print("kernel dispatches (durations in us):")
    print(f"  {'count':>6} {'avg':>10} {'min':>10} {'max':>10} {'total_ms':>10}  name")
    for name, d in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        print(f"  {len(d):6d} {sum(d)/len(d):10.2f} {min(d):10.2f} {max(d):10.2f} {sum(d)/1e3:10.3f}  {name[:110]}")
    by_grid = collections.OrderedDict()
    for name, g, s, e in _kernels_grid(db):
        if match in name:
            by_grid.setdefault((name, g), []).append((e - s) / 1e3)
    print(f"'{match}' dispatches by grid size (one kernel serves products of several shapes; durations in us):")
    print(f"  {'count':>6} {'avg':>10} {'min':>10} {'max':>10} {'total_ms':>10} {'grid_x':>9}  name")
    for (name, g), d in sorted(by_grid.items(), key=lambda kv: -sum(kv[1])):
        print(f"  {len(d):6d} {sum(d)/len(d):10.2f} {min(d):10.2f} {max(d):10.2f} {sum(d)/1e3:10.3f} {g:9d}  "
              f"{name[:90]}")
    cps = _copies(db)
    if not cps:
        return
    by = collections.defaultdict(list)
    for name, s, e, size in cps:
        by[(name, size)].append((e - s) / 1e3)
    print("memory copies (durations in us):")
    for (name, size), d in sorted(by.items()):
        gbs = size / (sum(d) / len(d) * 1e-6) / 1e9
        print(f"  {len(d):6d} x {size:>11d} B  avg {sum(d)/len(d):9.2f}  ({gbs:6.1f} GB/s each)  {name}")
    busy = _union([(s, e) for name, s, e in ks if match in name])
    tot = hid = 0.0
    for name, s, e, size in cps:
        if "DEVICE_TO_DEVICE" not in name:
            continue
        tot += e - s
        for a, b in busy:
            if b <= s:
                continue
            if a >= e:
                break
            hid += min(e, b) - max(s, a)
    if tot > 0:
        print(f"device-to-device copy time overlapped by '{match}' kernels: {100.0 * hid / tot:.1f}% "
              f"of {tot / 1e6:.3f} ms")


def _pmc(db, counter, grid=None):
    c = sqlite3.connect(db)
    per = collections.defaultdict(float)
    names = {}
    grids = dict(c.execute("select dispatch_id, grid_size_x from rocpd_kernel_dispatch"))
    for name, disp, cname, val in c.execute(
            "select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if cname.startswith(counter) and (grid is None or grids.get(disp) == grid or "calib" == name):
            per[disp] += val
            names[disp] = name
    out = collections.defaultdict(list)
    for disp, v in per.items():
        out[names[disp]].append(v)
    return out


def traffic(fetch_db, write_db, kernel, calib_kernel, calib_bytes, grid=None):
    f, fc_all = _pmc(fetch_db, "FETCH_SIZE", grid), _pmc(fetch_db, "FETCH_SIZE")
    w, wc_all = _pmc(write_db, "WRITE_SIZE", grid), _pmc(write_db, "WRITE_SIZE")

    def avg(d, match):
        vals = [v for n, vs in d.items() if match in n for v in vs]
        return sum(vals) / len(vals) if vals else None, len(vals)

    fk, nf = avg(f, kernel)
    wk, nw = avg(w, kernel)
    fc, _ = avg(fc_all, calib_kernel)
    wc, _ = avg(wc_all, calib_kernel)
    if None in (fk, wk, fc, wc):
        print("missing dispatches for the kernel or the calibration copy", file=sys.stderr)
        return 1
    sf = calib_bytes / (fc * 1024.0)
    sw = calib_bytes / (wc * 1024.0)
    print(f"calibration copy: FETCH_SIZE {fc:.0f} KiB, WRITE_SIZE {wc:.0f} KiB for {calib_bytes} B each way "
          f"-> scale {sf:.4f} (fetch), {sw:.4f} (write)")
    fb, wb = fk * 1024.0 * sf, wk * 1024.0 * sw
    gtxt = "" if grid is None else f" (grid_x {grid})"
    print(f"kernel '{kernel}'{gtxt}: {nf} fetch / {nw} write dispatches; per dispatch FETCH {fk:.0f} KiB, "
          f"WRITE {wk:.0f} KiB -> {fb/1e6:.2f} MB read + {wb/1e6:.2f} MB written = {(fb+wb)/1e6:.2f} MB")
    print(f"traffic_bytes_per_launch: {fb + wb:.0f}")
    return 0


def counters(db, match, simds=1024, xcds=8):
    c = sqlite3.connect(db)
    vals = collections.defaultdict(dict)
    names = {}
    for name, disp, cname, val in c.execute(
            "select name, dispatch_id, counter_name, counter_value from pmc_events"):
        vals[disp][cname] = vals[disp].get(cname, 0.0) + val
        names[disp] = name
    dur = {}
    try:
        for disp, s, e in c.execute("select dispatch_id, start, end from kernels"):
            dur[disp] = (e - s) * 1e-9
    except sqlite3.OperationalError:
        pass
    per = collections.defaultdict(list)
    for disp, v in vals.items():
        if match in names[disp]:
            per[names[disp]].append((disp, v))

    def med(xs):
        xs = sorted(x for x in xs if x is not None)
        return xs[len(xs) // 2] if xs else float("nan")

    for name, rows in sorted(per.items(), key=lambda kv: -len(kv[1])):
        d = [dur.get(k) for k, _ in rows]
        g = [v.get("GRBM_GUI_ACTIVE", 0.0) / xcds for _, v in rows]
        clk = med([gg / dd / 1e9 if gg and dd else None for gg, dd in zip(g, d)])
        busy = med([v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gg * simds) if gg else None
                    for gg, (_, v) in zip(g, rows)])
        wait = med([v.get("SQ_WAIT_ANY", 0.0) / v["SQ_WAVE_CYCLES"] if v.get("SQ_WAVE_CYCLES") else None
                    for _, v in rows])
        lds = med([v.get("SQ_LDS_BANK_CONFLICT", 0.0) / v["SQ_LDS_IDX_ACTIVE"] if v.get("SQ_LDS_IDX_ACTIVE") else None
                   for _, v in rows])
        print(f"  {name[:70]}: {len(rows)} dispatches, {med(d) * 1e6:.1f} us, clk {clk:.2f} GHz, "
              f"mfma_busy {100 * busy:.1f}%, WAIT_ANY {100 * wait:.1f}%, ldsconf {100 * lds:.1f}%")


def insts(db, match):
    c = sqlite3.connect(db)
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for name, disp, cname, val in c.execute(
            "select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if match in name:
            vals[disp][cname] += val
            names[disp] = name
    per = collections.defaultdict(list)
    for disp, v in vals.items():
        per[names[disp]].append(v)

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2]

    for name, rows in sorted(per.items(), key=lambda kv: -len(kv[1])):
        mfma = med([v.get("SQ_INSTS_MFMA", 0.0) for v in rows])
        if mfma <= 0:
            print(f"  {name[:70]}: {len(rows)} dispatches, no MFMA instructions")
            continue
        ratio = {k: med([v.get(f"SQ_INSTS_{k}", 0.0) for v in rows]) / mfma for k in ("VALU", "LDS", "VALU_TRANS_F32")}
        print(f"  {name[:70]}: {len(rows)} dispatches, per MFMA instruction: VALU {ratio['VALU']:.2f}, "
              f"LDS {ratio['LDS']:.2f}, transcendental {ratio['VALU_TRANS_F32']:.2f}")


def _pass_medians(db, match):
    c = sqlite3.connect(db)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for name, disp, cname, val in c.execute(
            "select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if match in name:
            per[disp][cname] += val
    dur = {d: (e - s) * 1e-9 for d, s, e in c.execute("select dispatch_id, start, end from kernels")}
    disps = sorted(per)
    if not disps:
        raise SystemExit(f"{db}: no dispatch of {match}")

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2]

    m = {cn: med([per[d][cn] for d in disps]) for cn in per[disps[0]]}
    m["_dur"] = med([dur[d] for d in disps])
    m["_n"] = len(disps)
    m["_cyc"] = m["GRBM_GUI_ACTIVE"] / 8
    return m


def requests(dbs, match, cus=256):
    p1, p2, p3, p4 = (_pass_medians(db, match) for db in dbs)
    req = p4["TCP_TCC_READ_REQ"]
    print(f"  dispatches {p4['_n']}, duration under counters {p4['_dur'] * 1e6:.0f} us, "
          f"clock {p4['_cyc'] / p4['_dur'] / 1e9:.2f} GHz")
    print(f"  TCP -> L2 read requests {req:.4g} ({req * 128 / 1e9:.2f} GB at 128 B)")
    print(f"  L2 hit rate {p4['TCC_HIT'] / (p4['TCC_HIT'] + p4['TCC_MISS']):.3f}, miss requests to the "
          f"fabric {p4['TCC_EA0_RDREQ']:.3g} ({p4['TCC_EA0_RDREQ'] * 128 / 1e9:.1f} GB)")
    print(f"  average TCP -> L2 read latency {p4['TCP_TCC_READ_REQ_LATENCY'] / req:.0f} cycles, "
          f"average L2 miss latency {p4['TCC_EA0_RDREQ_LEVEL'] / p4['TCC_EA0_RDREQ']:.0f} cycles")
    print(f"  TCP -> L2 reads in flight per CU {p4['TCP_TCC_READ_REQ_LATENCY'] / (p4['_cyc'] * cus):.1f}")
    print(f"  TCP stalled on pending misses {p3['TCP_PENDING_STALL_CYCLES'] / (p3['_cyc'] * cus):.2f} of cycles per CU")
    print(f"  TD busy {p2['TD_TD_BUSY'] / (p2['_cyc'] * cus):.2f}, stalled on the L1 "
          f"{p2['TD_TC_STALL'] / (p2['_cyc'] * cus):.2f}, TA busy {p2['TA_TA_BUSY'] / (p2['_cyc'] * cus):.2f} "
          f"of cycles per CU")
    print(f"  LDS data FIFO full {p1['SQ_LDS_DATA_FIFO_FULL']:.0f} cycles, waves waiting on LDS "
          f"{p1['SQ_WAIT_INST_LDS'] / p1['SQ_WAVE_CYCLES']:.2f} of wave cycles")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--match", default="gemm_kernel")
    r = sub.add_parser("traffic")
    r.add_argument("fetch_db")
    r.add_argument("write_db")
    r.add_argument("--kernel", required=True)
    r.add_argument("--calib-kernel", required=True)
    r.add_argument("--calib-bytes", type=float, required=True)
    r.add_argument("--grid", type=int, default=None, help="only dispatches with this grid_size_x")
    k = sub.add_parser("counters")
    k.add_argument("db")
    k.add_argument("--match", default="gemm_kernel")
    n = sub.add_parser("insts")
    n.add_argument("db")
    n.add_argument("--match", default="attn")
    q = sub.add_parser("requests")
    q.add_argument("dbs", nargs=4)
    q.add_argument("--match", default="gemm_kernel")
    a = ap.parse_args(argv)
    if a.cmd == "requests":
        requests(a.dbs, a.match)
        return 0
    if a.cmd == "insts":
        insts(a.db, a.match)
        return 0
    if a.cmd == "trace":
        trace(a.db, a.match)
        return 0
    if a.cmd == "counters":
        counters(a.db, a.match)
        return 0
    return traffic(a.fetch_db, a.write_db, a.kernel, a.calib_kernel, a.calib_bytes, a.grid)


if __name__ == "__main__":
    sys.exit(main())
