"""Turn rocprofv3 output into the figures the benchmark reports.

    python -m dynamic_moe_task_amd.profiling stats KERNEL_STATS_CSV
        Markdown table of a `--kernel-trace --stats` run (calls, average and
        total duration per kernel).

    python -m dynamic_moe_task_amd.profiling mfma COUNTER_CSV KERNEL_TRACE_CSV [--kernel REGEX]
        Matrix-core use per kernel from one `--pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
        SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE` run: bf16
        MFMA FLOPs (512 per MOP), their rate over the dispatch's duration
        against the 2.5 PF peak, and the fraction of SIMD cycles the matrix
        cores were busy (GRBM_GUI_ACTIVE summed over the 8 XCDs; 256 CUs of 4
        SIMDs), with the shader clock that GRBM_GUI_ACTIVE implies.

    python -m dynamic_moe_task_amd.profiling traffic --key decode/static \\
        --kernel moe_persistent --fetch A.csv --write B.csv \\
        --copy-fetch C.csv --copy-write D.csv --copy-bytes N --copy-kernel neg \\
        --out profiles/traffic.json
        HBM bytes per launch of the matched kernel from two `--pmc` runs
        (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by
        what the same counter reads for a plain copy kernel that moves a
        known number of bytes.  The result is merged into the JSON file under
        `key`.

Host-side text processing only; nothing here touches the GPU.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import re
import statistics
import sys


CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def kernel_source_digest():
    """Digest of the device sources; traffic figures taken from another
    digest describe a kernel that has since changed."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in columns {list(row)}")


def counter_per_dispatch(path, counter, kernel_regex):
    """Values of `counter` (summed over its instances) for every dispatch
    whose kernel name matches `kernel_regex`, in dispatch order."""
    rx = re.compile(kernel_regex)
    by_dispatch = {}
    for r in read_csv(path):
        if _col(r, "Counter_Name") != counter:
            continue
        name = _col(r, "Kernel_Name")
        if not rx.search(name):
            continue
        d = int(_col(r, "Dispatch_Id", "Correlation_Id"))
        by_dispatch[d] = by_dispatch.get(d, 0.0) + float(_col(r, "Counter_Value"))
    return [by_dispatch[d] for d in sorted(by_dispatch)]


def traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, kernel_regex, copy_regex,
            skip_first=1):
    """HBM bytes per launch (median over dispatches, the first `skip_first`
    dropped as warm-up) with each counter scaled so that the copy kernel's
    reading equals the bytes it is known to move."""
    cf = counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", copy_regex)
    cw = counter_per_dispatch(copy_write_csv, "WRITE_SIZE", copy_regex)
    mf = counter_per_dispatch(fetch_csv, "FETCH_SIZE", kernel_regex)
    mw = counter_per_dispatch(write_csv, "WRITE_SIZE", kernel_regex)
    for name, v in (("copy FETCH_SIZE", cf), ("copy WRITE_SIZE", cw), ("FETCH_SIZE", mf), ("WRITE_SIZE", mw)):
        if not v:
            raise ValueError(f"no {name} dispatches matched")
    med = lambda v: statistics.median(v[skip_first:] if len(v) > skip_first else v)  # noqa: E731
    f_scale = copy_bytes / (med(cf) * 1024.0)
    w_scale = copy_bytes / (med(cw) * 1024.0)
    fetch = med(mf) * 1024.0 * f_scale
    write = med(mw) * 1024.0 * w_scale
    return {"fetch_bytes": round(fetch), "write_bytes": round(write), "total_bytes": round(fetch + write),
            "fetch_kib_raw": med(mf), "write_kib_raw": med(mw), "fetch_scale": round(f_scale, 4),
            "write_scale": round(w_scale, 4), "dispatches": [len(mf), len(mw)],
            "copy_bytes": copy_bytes, "source_digest": kernel_source_digest()}


def mfma_table(counter_csv, trace_csv, kernel_regex=".", xcds=8, cus=256, simds=4, peak_tfs=2500.0):
    """Per kernel (median over its dispatches): duration, bf16 MFMA TFLOP/s
    and fraction of peak, MFMA busy fraction of all SIMD cycles, clock."""
    rx = re.compile(kernel_regex)
    dur, names = {}, {}
    for r in read_csv(trace_csv):
        d = int(_col(r, "Dispatch_Id", "Correlation_Id"))
        dur[d] = (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3
        names[d] = _col(r, "Kernel_Name")
    per = {}
    for r in read_csv(counter_csv):
        d = int(_col(r, "Dispatch_Id", "Correlation_Id"))
        name = _col(r, "Kernel_Name")
        if not rx.search(name):
            continue
        per.setdefault(d, {"name": name})
        c = _col(r, "Counter_Name")
        per[d][c] = per[d].get(c, 0.0) + float(_col(r, "Counter_Value"))
    by_kernel = {}
    for d, v in per.items():
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" not in v or d not in dur or v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] == 0:
            continue
        us = dur[d]
        flops = v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
        cyc = v.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * cus * simds) if cyc else float("nan")
        by_kernel.setdefault(v["name"], []).append((us, flops, flops / (us * 1e-6) / 1e12, busy, cyc / us / 1e3))
    out = ["| kernel | dispatches | µs | bf16 GFLOP | TFLOP/s | of 2.5 PF | MFMA busy | clock GHz |",
           "|---|---|---|---|---|---|---|---|"]
    for name, rows in by_kernel.items():
        med = lambda i: statistics.median(r[i] for r in rows)  # noqa: E731
        out.append(f"| `{name[:70]}` | {len(rows)} | {med(0):.1f} | {med(1) / 1e9:.1f} | {med(2):.1f} | "
                   f"{med(2) / peak_tfs:.3f} | {med(3):.3f} | {med(4):.2f} |")
    return "\n".join(out)


def stats_table(path, top=12):
    rows = read_csv(path)
    out = ["| kernel | calls | avg µs | min µs | max µs | total µs | % |", "|---|---|---|---|---|---|---|"]
    for r in rows[:top]:
        name = _col(r, "Name", "KERNEL_NAME", "Kernel_Name")
        calls = int(_col(r, "Calls"))
        to_us = lambda k: float(_col(r, k)) / 1e3  # noqa: E731  (ns -> µs)
        out.append(f"| `{name[:90]}` | {calls} | {to_us('AverageNs'):.2f} | {to_us('MinNs'):.2f} | "
                   f"{to_us('MaxNs'):.2f} | {to_us('TotalDurationNs'):.1f} | {float(_col(r, 'Percentage')):.1f} |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--top", type=int, default=12)
    m = sub.add_parser("mfma")
    m.add_argument("counters")
    m.add_argument("trace")
    m.add_argument("--kernel", default=".")
    t = sub.add_parser("traffic")
    t.add_argument("--key", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--copy-kernel", default="neg")
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.csv, a.top))
        return 0
    if a.cmd == "mfma":
        print(mfma_table(a.counters, a.trace, a.kernel))
        return 0
    res = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, a.kernel, a.copy_kernel)
    data = {}
    if os.path.exists(a.out):
        with open(a.out) as f:
            data = json.load(f)
    data[a.key] = res
    with open(a.out, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({a.key: res}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
