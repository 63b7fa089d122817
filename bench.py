"""Benchmark: one MoE layer (Qwen3-30B-A3B-shaped, 128 experts, top-8) on one
MI355X through the C ABI.  A step is one launch of the whole hot path
(router, top-k, scan, dispatch, gate/up+SwiGLU, down, combine) over one batch
of synthetic tokens already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]
                    [--sched ordered] [--copies R] [--no-cpu] [--traffic FILE]

Prints ONE JSON line.  `value` is tokens/s of the chosen schedule; the other
schedules, µs/layer and the roofline fraction ride along in the same line.
Weights are rotated over R device copies so that consecutive steps do not
reuse expert weights left in the 256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFS = 2500.0      # MI355X dense bf16 MFMA, published

METRIC = "µs per MoE layer & tokens/s at 1 MI355X; %HBM peak (decode) / %MFMA (batch 256)"
# live schedules, persistent ones first; the dynamic push/pop schedule is
# switched off in the library
SCHEDS = ("static", "ordered", "barrier", "kbk")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill_zipf", "tiny", "decoder", "tokens", "mlp"],
                    help="decoder: only the decoder-layer section; tokens: only the token-count table at "
                         "--counts; mlp: only the dense-MLP table (diagnostics and profiling)")
    ap.add_argument("--mlps", default="", help="indices into the dense-MLP table for --workload mlp (default all)")
    ap.add_argument("--counts", default="1,128,1024,4096", help="token counts of --workload tokens")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload's layer at this many tokens instead of its own T (diagnostics, "
                         "e.g. a per-task trace at T=1)")
    ap.add_argument("--sched", default="ordered", choices=list(SCHEDS),
                    help="schedule behind `value` (the others are timed alongside)")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated over steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured with rocprofv3 counters (JSON)")
    ap.add_argument("--only-sched", action="store_true", help="time only --sched (for profiling)")
    ap.add_argument("--trace", default="", help="write a per-task trace summary of each persistent "
                    "schedule to this JSON file (one extra traced launch each, outside the timing); the raw "
                    "records go next to it as .npz")
    ap.add_argument("--repeat", type=int, default=3, help="timing loops per schedule; the median is reported")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the prefill (T=256, Zipf-biased) and batch-size-sweep measurements")
    ap.add_argument("--sweep-steps", type=int, default=200)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="calibration only: run a plain elementwise copy (read N MiB, write N MiB) --steps "
                         "times and exit; its HBM counters scale the MoE kernel's")
    return ap.parse_args()


def copy_calibration(mib, steps):
    """A plain device copy of known size (torch.neg over bf16: reads and
    writes `mib` MiB per launch), for scaling rocprofv3's FETCH_SIZE and
    WRITE_SIZE readings to bytes."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.randn(n, device="cuda").to(torch.bfloat16)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        torch.neg(src, out=dst)
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / steps
    nbytes = mib * (1 << 20)
    print(json.dumps({"copy_read_bytes": nbytes, "copy_write_bytes": nbytes, "us_per_launch": round(us, 2),
                      "GBps": round(2 * nbytes / (us * 1e-6) / 1e9, 1)}))


TASK_NAMES = {1: "R", 2: "K", 3: "S", 4: "D", 5: "G1", 6: "G2", 7: "C", 8: "L",  # L: LDS routing tables
              9: "N1", 10: "QKV", 11: "ATT", 12: "ATTC", 13: "O", 14: "N2",  # the decoder's attention block
              15: "WG"}  # per workgroup: wait = entry to counter set known, body = task lists, notify = exit


def tile_rows(counts, bm=64):
    """Rows of each row tile, in the kernel's numbering: tiles of more than
    32 rows (four 16-row MFMA blocks) first, then of 17-32 rows, then of at
    most 16, each class in expert order; expert e with c rows has c // bm
    full tiles and one tile of the remainder (measurement bookkeeping)."""
    four, two, one = [], [], []
    for c in (int(x) for x in counts):
        full, rem = divmod(c, bm)
        four += [bm] * full
        if rem > 32:
            four.append(rem)
        elif rem > 16:
            two.append(rem)
        elif rem > 0:
            one.append(rem)
    return four + two + one


def tile_mfma(rec_typ, rec_a, body_us, rows, H, I, grid, bn1, bn2):
    """Tile-level MFMA use of the G tasks whose row tile has four row blocks
    (33-64 rows): the tile's FLOPs over its body time, against the
    workgroup's share of the bf16 peak (the grid shares the chip evenly)."""
    peak_wg = BF16_PEAK_TFS * 1e12 / grid
    out = {}
    for t, name, cols, kdim in ((5, "G1", 2 * bn1, H), (6, "G2", bn2, I)):
        m = rec_typ == t
        r = np.array([rows[a] if a < len(rows) else 0 for a in rec_a[m]])
        big = r > 32
        if not big.any():
            continue
        flops = 2.0 * r[big] * cols * kdim
        eff = flops / (body_us[m][big] * 1e-6) / peak_wg
        wbytes = cols * kdim * 2
        out[name] = {"tiles": int(big.sum()), "rows_mean": round(float(r[big].mean()), 1),
                     "body_us_mean": round(float(body_us[m][big].mean()), 2),
                     "mfma_frac_mean": round(float(eff.mean()), 4),
                     "flop_per_weight_byte": round(float(flops.mean() / wbytes), 1)}
    return out


def trace_summary(bufs, T, sched, khz, stream_ptr, records=1 << 16, dump=None, shape=None, launch=None):
    """One traced launch: per task type, count, mean/max duration, mean
    wait, and the first start / last end in µs from the earliest wait; with
    `shape`, the tile-level MFMA use of the four-block G tiles.  `launch`
    (given the trace buffer) replaces the MoE layer launch (the decoder)."""
    import torch
    from dynamic_moe_task_amd import binding as B
    tr = torch.zeros(B.trace_words(records), dtype=torch.int32, device="cuda")
    if launch is not None:
        B.check(launch(tr))
    else:
        B.check(B.moe_layer_launch(bufs.desc, T, bufs.args(trace=tr), B.SCHEDS[sched], stream_ptr))
    B.check(B.etc_sync(stream_ptr))
    raw = tr.cpu().numpy().view(np.uint32)
    allrec = raw[16:16 + 8 * records].reshape(records, 8)
    rec = allrec[allrec[:, 0] != 0]  # each workgroup fills its own slots; unused ones stay zero
    n = len(rec)
    if dump:
        np.savez(dump, raw=np.concatenate([raw[:16], rec.reshape(-1)]), khz=khz)
    rec = rec.astype(np.int64)
    wg, typ = rec[:, 0] & 0xFFFFFF, rec[:, 0] >> 24
    tw = (rec[:, 4] << 32) | rec[:, 3]

    def unwrap(lo):  # the later stamps share tw's high word unless they wrapped
        t = (rec[:, 4] << 32) | lo
        return np.where(t < tw, t + (1 << 32), t)

    ts, tb, te = unwrap(rec[:, 5]), unwrap(rec[:, 6]), unwrap(rec[:, 7])
    t0 = tw.min()
    us = 1e3 / khz
    out = {"records": n, "span_us": round(float((te.max() - t0) * us), 2)}
    for t, name in TASK_NAMES.items():
        m = typ == t
        if not m.any():
            continue
        body = (tb[m] - ts[m]) * us
        notify = (te[m] - tb[m]) * us
        wt = (ts[m] - tw[m]) * us
        out[name] = {"n": int(m.sum()), "body_mean_us": round(float(body.mean()), 2),
                     "body_max_us": round(float(body.max()), 2),
                     "notify_mean_us": round(float(notify.mean()), 2),
                     "wait_mean_us": round(float(wt.mean()), 2), "wait_max_us": round(float(wt.max()), 2),
                     "first_start_us": round(float((ts[m].min() - t0) * us), 2),
                     "last_end_us": round(float((te[m].max() - t0) * us), 2)}
    per_wg = np.bincount(wg, weights=(te - ts) * us)
    out["busy_per_wg_us"] = {"mean": round(float(per_wg.mean()), 2), "max": round(float(per_wg.max()), 2)}
    if shape is not None:
        rows = tile_rows(bufs.counts.cpu().numpy())
        grid = int(raw[2])
        info = B.moe_layer_info(bufs.desc)
        out["tile_mfma_four_block"] = tile_mfma(typ, rec[:, 1], (tb - ts) * us, rows, shape.H, shape.I, grid,
                                                info.bn1_for(T, shape.k), info.bn2_for(T, shape.k))
    return out


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def time_sched(bufs, T, sched, steps, warmup, w13s, w2s, stream_ptr, per_launch=None):
    """Average µs per launch over `steps` back-to-back launches, bracketed by
    HIP events on the launch stream.  With a list `per_launch`, a second pass
    brackets every launch with its own pair of events and appends the
    per-launch µs to it (for the median and the p10/p90 spread)."""
    import torch
    from dynamic_moe_task_amd import binding as B
    R = len(w13s)
    args = [bufs.args(w13=w13s[i], w2=w2s[i]) for i in range(R)]
    code = B.SCHEDS[sched]
    for i in range(warmup):
        B.check(B.moe_layer_launch(bufs.desc, T, args[i % R], code, stream_ptr))
    B.check(B.etc_sync(stream_ptr))
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        B.check(B.moe_layer_launch(bufs.desc, T, args[i % R], code, stream_ptr))
    end.record()
    torch.cuda.synchronize()
    rc = B.etc_sync(stream_ptr)
    if rc != 0:
        raise B.EtcError(rc, B.etc_last_error())
    if per_launch is not None:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record()
            B.check(B.moe_layer_launch(bufs.desc, T, args[i % R], code, stream_ptr))
            evs[i][1].record()
        torch.cuda.synchronize()
        B.check(B.etc_sync(stream_ptr))
        per_launch += [a.elapsed_time(b) * 1e3 for a, b in evs]
    return start.elapsed_time(end) * 1e3 / steps


def dist(samples):
    """Median and p10 / p90 of per-launch µs."""
    x = np.asarray(samples, np.float64)
    return {"p10": round(float(np.percentile(x, 10)), 2), "median": round(float(np.median(x)), 2),
            "p90": round(float(np.percentile(x, 90)), 2), "n": int(x.size)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_oracle_rate(shape, w, X, seconds, threads):
    """Tokens/s of the oracle as it stands (plain C, fp64) on `threads`
    threads: whole layers for decode/tiny; for larger batches a bounded
    sample (routing for all T plus the expert rows of a token slice)."""
    import oracle
    k = shape.k
    used = oracle.set_threads(threads)
    t0 = time.perf_counter()
    n = 0
    toks = 0
    sample = ""
    step = 8 * max(1, used)
    while True:
        if shape.T <= 16:
            oracle.moe(X, w.Wr, w.W13, w.Wd, k=k, norm_topk=shape.norm_topk, bias=w.bias)
            toks += shape.T
            sample = f"whole layer, T={shape.T}, repeated"
        else:
            r = oracle.route(X, w.Wr, k, bias=w.bias)
            sub = np.arange(n * step % shape.T, n * step % shape.T + step, dtype=np.int32) % shape.T
            oracle.moe_tokens(sub, X, w.W13, w.Wd, r["topk_ids"], r["topk_w"])
            toks += len(sub)
            sample = f"routing of all {shape.T} tokens + expert rows of {step}-token slices, repeated"
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return toks / dt, used, f"{sample}; {n} calls in {dt:.1f} s"


def cpu_baseline(shape, w, X, seconds):
    """The oracle timed on this host's cores in the same run: one thread,
    then OpenMP over the rows on every core this process may use
    (sched_getaffinity, capped by OMP_NUM_THREADS when the host sets it).
    `value`/`cores` are the multi-core leg."""
    ncores = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        ncores = min(ncores, int(env))
    v1, _, s1 = cpu_oracle_rate(shape, w, X, seconds / 2, 1)
    vn, used, sn = cpu_oracle_rate(shape, w, X, seconds / 2, ncores)
    return {"value": vn, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{sn}; OpenMP over rows", "cpu_model": cpu_model(),
            "single_thread": {"value": v1, "unit": "tokens/s", "cores": 1, "sample": s1}}


RIDGE = BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)  # flop per byte where MFMA and HBM bounds meet


def measure_prefill(Wr, w13s, w2s, sp, steps, warmup, repeat, main_sched):
    """Prefill chunk: T=256 with the Zipf(1.1) logit bias (hot experts get
    most tokens, some get none).  Same expert weights as the decode layer."""
    import torch
    from dynamic_moe_task_amd import binding as B
    from dynamic_moe_task_amd import workloads as wl
    shape = wl.PREFILL_ZIPF
    T = shape.T
    X = wl.make_tokens(shape, T, 0)
    bias = torch.from_numpy(wl.zipf_bias(shape, 0)).cuda()
    desc = B.moe_desc(T, shape.H, shape.E, shape.k, shape.I, shape.norm_topk, True)
    bufs = B.MoELayerBuffers.allocate(desc, Wr, w13s[0], w2s[0], bias)
    bufs.x[:T].copy_(dev_bf16(X))
    B.check(B.moe_layer_launch(desc, T, bufs.args(), B.SCHEDS["static"], sp))
    B.check(B.etc_sync(sp))
    counts = bufs.counts.cpu().numpy()
    n_act = int((counts > 0).sum())
    alg_bytes = wl.algorithmic_bytes(shape, T, n_act)
    alg_flops = wl.algorithmic_flops(shape, T)
    runs = {s: [] for s in SCHEDS}
    for _ in range(repeat):  # interleaved, then medians
        for sch in SCHEDS:
            runs[sch].append(time_sched(bufs, T, sch, steps, warmup, w13s, w2s, sp))
    us = {s: float(np.median(v)) for s, v in runs.items()}
    best = min(us.values())
    ai = alg_flops / alg_bytes
    m = us[main_sched]
    return {
        "workload": shape.name, "T": T, "active_experts": n_act, "max_expert_tokens": int(counts.max()),
        "us_per_layer": {k: round(v, 2) for k, v in us.items()},
        "schedule": main_sched,
        "tokens_per_s": round(T / (m * 1e-6), 1),
        "algorithmic_bytes": alg_bytes, "algorithmic_flops": alg_flops,
        "hbm_frac": round(alg_bytes / (m * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
        "mfma_frac_whole_layer": round(alg_flops / (m * 1e-6) / (BF16_PEAK_TFS * 1e12), 5),
        "mfma_frac_cap": round(ai / RIDGE, 4),
        "note": "whole-layer MFMA use is capped at AI/ridge: at this batch the layer is HBM-bound",
        "fastest": min(us, key=us.get), "fastest_us": round(best, 2),
    }


def measure_sweep(Wr, w13s, w2s, sp, steps, main_sched):
    """Shape dynamism: one template (T_max=512), batch B ~ U{1..512} per step,
    fresh tokens each step; per-launch latency from HIP events."""
    import torch
    from dynamic_moe_task_amd import binding as B
    from dynamic_moe_task_amd import workloads as wl
    shape = wl.SWEEP
    Bs = wl.sweep_batches(0, steps)
    desc = B.moe_desc(shape.T, shape.H, shape.E, shape.k, shape.I, shape.norm_topk, False)
    bufs = B.MoELayerBuffers.allocate(desc, Wr, w13s[0], w2s[0], None)
    xs = [dev_bf16(wl.sweep_tokens(shape, i, int(b), 0)) for i, b in enumerate(Bs)]
    R = len(w13s)
    args = [bufs.args(x=xs[i], w13=w13s[i % R], w2=w2s[i % R]) for i in range(steps)]
    code = B.SCHEDS[main_sched]
    for i in range(3):  # warm-up launches at a few sizes
        B.check(B.moe_layer_launch(desc, int(Bs[i]), args[i], code, sp))
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        B.check(B.moe_layer_launch(desc, int(Bs[i]), args[i], code, sp))
        evs[i][1].record()
    torch.cuda.synchronize()
    B.check(B.etc_sync(sp))
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    small = Bs <= 64
    return {
        "steps": steps, "B_min": int(Bs.min()), "B_max": int(Bs.max()), "schedule": main_sched,
        "us_p50": round(float(np.percentile(us, 50)), 2), "us_p90": round(float(np.percentile(us, 90)), 2),
        "us_p99": round(float(np.percentile(us, 99)), 2), "us_max": round(float(us.max()), 2),
        "us_p50_B_le_64": round(float(np.median(us[small])), 2) if small.any() else None,
        "tokens_per_s": round(float(Bs.sum() / (us.sum() * 1e-6)), 1),
        "recompiles": 0, "graph_captures": 0, "code_objects": 1,
    }


def measure_token_counts(Wr, w13s, w2s, sp, steps, warmup, repeat, counts=(1, 128, 1024, 4096)):
    """The pages compare schedules on the same MoE layer at several token
    counts (Event Tensor paper, Table 2).  Same Qwen3-30B-A3B shape, no bias;
    µs per layer of each schedule, and the speed-ups of the two event-driven
    megakernel schedules over the barrier megakernel and over KBK."""
    import torch
    from dynamic_moe_task_amd import binding as B
    from dynamic_moe_task_amd import workloads as wl
    shape = wl.DECODE
    out = {}
    for T in counts:
        X = wl.make_tokens(shape, T, 0)
        desc = B.moe_desc(T, shape.H, shape.E, shape.k, shape.I, shape.norm_topk, False)
        bufs = B.MoELayerBuffers.allocate(desc, Wr, w13s[0], w2s[0], None)
        bufs.x[:T].copy_(dev_bf16(X))
        runs = {s: [] for s in SCHEDS}
        for _ in range(repeat):
            for s in SCHEDS:
                runs[s].append(time_sched(bufs, T, s, steps, warmup, w13s, w2s, sp))
        us = {s: float(np.median(v)) for s, v in runs.items()}
        row = {"us_per_layer": {s: round(v, 2) for s, v in us.items()}}
        # whole-layer MFMA use of the ORDERED megakernel (the layer's
        # algorithmic FLOPs over its time, against the bf16 peak)
        row["ordered_mfma_frac_whole_layer"] = round(
            wl.algorithmic_flops(shape, T) / (us["ordered"] * 1e-6) / (BF16_PEAK_TFS * 1e12), 5)
        for s in ("static", "ordered"):
            row[f"{s}_over_barrier_speedup"] = round(us["barrier"] / us[s], 3)
            row[f"{s}_over_kbk_speedup"] = round(us["kbk"] / us[s], 3)
        out[f"T={T}"] = row
        del bufs
        torch.cuda.synchronize()
    return out


def measure_dense_mlps(sp, steps, warmup, repeat, which=None, trace=""):
    """The dense MLPs of the pages' appendix table (S = 8192 tokens) run
    through the MoE path as one expert (E = 1, k = 1): the big-tile grouped
    GEMM with full 256-row tiles.  µs per layer (ORDERED and kernel by
    kernel), TFLOP/s and the fraction of the 2.5 PF bf16 MFMA peak.  For
    context (not the product path): the layer's two GEMMs alone through
    torch.matmul (hipBLASLt), without routing, SwiGLU or combine."""
    import torch
    from dynamic_moe_task_amd import binding as B
    from dynamic_moe_task_amd import workloads as wl
    out = {}
    for i, shape in enumerate(wl.MLP_TABLE):
        if which is not None and i not in which:
            continue
        w = wl.make_weights(shape, 0)
        W13, Wd = dev_bf16(w.W13), dev_bf16(w.Wd)
        X = wl.make_tokens(shape, shape.T, 0)
        desc = B.moe_desc(shape.T, shape.H, shape.E, shape.k, shape.I, True, False)
        bufs = B.MoELayerBuffers.allocate(desc, dev_bf16(w.Wr), W13, Wd, None)
        bufs.x[:shape.T].copy_(dev_bf16(X))
        flops = wl.algorithmic_flops(shape, shape.T)
        row = {"S": shape.T, "H": shape.H, "I": shape.I, "gflop": round(flops / 1e9, 1), "us_per_layer": {}}
        for sched in ("ordered", "kbk"):
            us = float(np.median([time_sched(bufs, shape.T, sched, steps, warmup, [W13], [Wd], sp)
                                  for _ in range(repeat)]))
            row["us_per_layer"][sched] = round(us, 1)
        if trace:
            khz = B.moe_layer_info(desc).wall_clock_khz
            base = os.path.splitext(trace)[0]
            row["trace_ordered"] = trace_summary(bufs, shape.T, "ordered", khz, sp, dump=f"{base}_mlp{i + 1}.npz")
        best = min(row["us_per_layer"].values())
        row["tflops"] = round(flops / (best * 1e-6) / 1e12, 1)
        row["mfma_frac"] = round(flops / (best * 1e-6) / (BF16_PEAK_TFS * 1e12), 4)
        # hipBLASLt reference: x W13^T (2I columns) and h Wd^T, contiguous operands
        xa = bufs.x[:shape.T]
        w13t = W13[0].t().contiguous()
        wdt = Wd[0].t().contiguous()
        hm = torch.empty(shape.T, shape.I, dtype=torch.bfloat16, device="cuda")

        def gemms():
            torch.matmul(xa, w13t)
            torch.matmul(hm, wdt)

        for _ in range(warmup):
            gemms()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            gemms()
        e1.record()
        torch.cuda.synchronize()
        lib_us = e0.elapsed_time(e1) * 1e3 / steps
        row["hipblaslt_two_gemms_us"] = round(lib_us, 1)
        row["hipblaslt_mfma_frac"] = round(6.0 * shape.T * shape.H * shape.I / (lib_us * 1e-6) / (BF16_PEAK_TFS * 1e12), 4)
        out[shape.name.split()[0]] = row
        del bufs, W13, Wd, w13t, wdt, hm
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def measure_decoder(Wr, w13s, w2s, sp, steps, warmup, repeat, scheds=("static", "ordered", "kbk"), trace=""):
    """The decoder layer around the MoE layer as one persistent kernel
    (batch 8, 32 query / 4 kv heads of 128, 4096 cached entries per
    sequence, then the same MoE block with the decode weights), against its
    HBM floor, and kernel by kernel."""
    import torch
    from dynamic_moe_task_amd import binding as B
    from dynamic_moe_task_amd import workloads as wl
    s = wl.DECODER
    w, X, kc, vc = wl.make_decoder(s, 0, moe=wl.MoEWeights(None, None, None))
    desc = B.decoder_desc(s.T, s.H, s.nq, s.nkv, s.d, s.Lcap, s.moe.E, s.moe.k, s.moe.I, s.theta, s.eps)
    kcd, vcd = dev_bf16(kc), dev_bf16(vc)
    bufs = B.DecoderBuffers.allocate(desc, dev_bf16(w.g1), dev_bf16(w.Wqkv), dev_bf16(w.Wo), dev_bf16(w.g2), kcd, vcd,
                                     Wr, w13s[0], w2s[0])
    bufs.x[:s.T].copy_(dev_bf16(X))
    B.check(B.decoder_layer_launch(desc, s.T, s.pos, bufs.args(), B.SCHEDS["static"], sp))
    B.check(B.etc_sync(sp))
    n_act = int((bufs.moe.counts.cpu().numpy() > 0).sum())
    alg = wl.decoder_algorithmic_bytes(s, n_act)
    R = len(w13s)
    args = [bufs.args(w13=w13s[i], w2=w2s[i]) for i in range(R)]

    def timed(sched):
        code = B.SCHEDS[sched]
        for i in range(warmup):
            B.check(B.decoder_layer_launch(desc, s.T, s.pos, args[i % R], code, sp))
        B.check(B.etc_sync(sp))
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            B.check(B.decoder_layer_launch(desc, s.T, s.pos, args[i % R], code, sp))
        end.record()
        torch.cuda.synchronize()
        B.check(B.etc_sync(sp))
        return start.elapsed_time(end) * 1e3 / steps

    runs = {x: [] for x in scheds}
    for _ in range(repeat):
        for x in scheds:
            runs[x].append(timed(x))
    us = {x: float(np.median(v)) for x, v in runs.items()}
    best = min((x for x in ("static", "ordered") if x in us), key=lambda x: us[x], default=scheds[0])
    if trace:
        khz = B.moe_layer_info(B.moe_desc(s.T, s.H, s.moe.E, s.moe.k, s.moe.I)).wall_clock_khz
        base = os.path.splitext(trace)[0]
        summ = {x: trace_summary(None, s.T, x, khz, sp, dump=f"{base}_{x}.npz",
                                 launch=lambda tr, x=x: B.decoder_layer_launch(desc, s.T, s.pos, bufs.args(trace=tr),
                                                                              B.SCHEDS[x], sp))
                for x in scheds if x != "kbk"}
        with open(trace, "w") as f:
            json.dump(summ, f, indent=1)
    return {
        "workload": s.name, "T": s.T, "pos": s.pos, "heads": [s.nq, s.nkv, s.d], "active_experts": n_act,
        "us_per_layer": {x: round(v, 2) for x, v in us.items()},
        "tokens_per_s": round(s.T / (us[best] * 1e-6), 1), "schedule": best,
        "algorithmic_bytes": alg, "hbm_floor_us": round(alg / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
        "hbm_frac": round(alg / (us[best] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
        "megakernel_over_kbk_speedup": round(us["kbk"] / us[best], 3) if "kbk" in us else None,
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    if a.copy_mib:
        copy_calibration(a.copy_mib, a.steps)
        return
    import torch
    from dynamic_moe_task_amd import binding as B
    from dynamic_moe_task_amd import workloads as wl

    if a.workload == "mlp":
        torch.cuda.set_device(0)
        sp = torch.cuda.current_stream().cuda_stream
        which = {int(v) for v in a.mlps.split(",")} if a.mlps else None
        print(json.dumps(measure_dense_mlps(sp, a.steps, a.warmup, a.repeat, which, a.trace)), flush=True)
        return
    if a.workload in ("decoder", "tokens"):
        import torch
        torch.cuda.set_device(0)
        w = wl.make_weights(wl.DECODE, 0)
        Wr, W13, Wd = dev_bf16(w.Wr), dev_bf16(w.W13), dev_bf16(w.Wd)
        R = max(1, a.copies)
        w13s = [W13] + [W13.clone() for _ in range(R - 1)]
        w2s = [Wd] + [Wd.clone() for _ in range(R - 1)]
        sp = torch.cuda.current_stream().cuda_stream
        if a.workload == "tokens":
            counts = tuple(int(v) for v in a.counts.split(","))
            print(json.dumps(measure_token_counts(Wr, w13s, w2s, sp, a.steps, a.warmup, a.repeat, counts)), flush=True)
            return
        scheds = (a.sched,) if a.only_sched else ("static", "ordered", "kbk")
        print(json.dumps(measure_decoder(Wr, w13s, w2s, sp, a.steps, a.warmup, a.repeat, scheds, a.trace)), flush=True)
        return
    shape = wl.SHAPES[a.workload]
    if a.tokens > 0:
        import dataclasses
        shape = dataclasses.replace(shape, T=a.tokens, name=f"{shape.name} at T={a.tokens}")
    T = shape.T
    w, X = wl.make_layer(shape, 0)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    Wr = dev_bf16(w.Wr)
    W13 = dev_bf16(w.W13)
    Wd = dev_bf16(w.Wd)
    bias = torch.from_numpy(w.bias).cuda() if w.bias is not None else None
    R = max(1, a.copies) if shape.E > 8 else 1
    w13s = [W13] + [W13.clone() for _ in range(R - 1)]
    w2s = [Wd] + [Wd.clone() for _ in range(R - 1)]
    xd = dev_bf16(X)
    torch.cuda.synchronize()

    # first-step warm-up: library load, workspace set-up and the first launch
    # (code-object load included) up to its completion, all on the host clock
    t_w0 = time.perf_counter()
    B.lib()
    desc = B.moe_desc(T, shape.H, shape.E, shape.k, shape.I, shape.norm_topk, bias is not None)
    bufs = B.MoELayerBuffers.allocate(desc, Wr, W13, Wd, bias)
    bufs.x[:T].copy_(xd)
    B.check(B.moe_layer_launch(desc, T, bufs.args(), B.SCHEDS[a.sched], sp))
    B.check(B.etc_sync(sp))
    warmup_ms = (time.perf_counter() - t_w0) * 1e3
    counts = bufs.counts.cpu().numpy()
    n_act = int((counts > 0).sum())
    alg_bytes = wl.algorithmic_bytes(shape, T, n_act)
    alg_flops = wl.algorithmic_flops(shape, T)

    scheds = [a.sched] if a.only_sched else list(SCHEDS)
    runs = {s: [] for s in scheds}
    per_launch = {s: [] for s in scheds}
    for _ in range(max(1, a.repeat)):  # interleave the schedules, then take medians
        for s in scheds:
            runs[s].append(time_sched(bufs, T, s, a.steps, a.warmup, w13s, w2s, sp, per_launch[s]))
    us = {s: float(np.median(v)) for s, v in runs.items()}
    us_main = us[a.sched]

    achieved_gbs = alg_bytes / (us_main * 1e-6) / 1e9
    # HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE (scaled by a
    # copy kernel of known size); null unless taken on the current sources
    traffic = None
    traffic_note = "no counter figures for this workload and schedule"
    if a.traffic and os.path.exists(a.traffic):
        from dynamic_moe_task_amd.profiling import kernel_source_digest
        with open(a.traffic) as f:
            tr = json.load(f).get(f"{a.workload}/{a.sched}")
        if tr is not None:
            if tr.get("source_digest") == kernel_source_digest():
                traffic = tr["total_bytes"]
                traffic_note = (f"fetch {tr['fetch_bytes']} B + write {tr['write_bytes']} B per launch "
                                f"(scales {tr['fetch_scale']}, {tr['write_scale']})")
            else:
                traffic_note = "counters were taken on different kernel sources"
    roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": f"moe_persistent<{a.sched}>" if a.sched != "kbk" else "kbk_* (6 launches)",
                "algorithmic_bytes": alg_bytes, "traffic_note": traffic_note}
    mfma_frac = alg_flops / (us_main * 1e-6) / (BF16_PEAK_TFS * 1e12)

    if a.trace:
        info = B.moe_layer_info(desc)
        base = os.path.splitext(a.trace)[0]
        summ = {s: trace_summary(bufs, T, s, info.wall_clock_khz, sp, dump=f"{base}_{s}.npz", shape=shape)
                for s in ("static", "ordered", "barrier")}
        summ["grid"] = info.grid
        with open(a.trace, "w") as f:
            json.dump(summ, f, indent=1)

    extra = {}
    if not a.no_extra and a.workload == "decode":
        extra["prefill_zipf"] = measure_prefill(Wr, w13s, w2s, sp, max(10, a.steps // 2), a.warmup, a.repeat,
                                                a.sched)
        extra["sweep"] = measure_sweep(Wr, w13s, w2s, sp, a.sweep_steps, a.sched)
        extra["token_counts"] = measure_token_counts(Wr, w13s, w2s, sp, max(10, a.steps // 2), a.warmup, a.repeat)
        extra["decoder_layer"] = measure_decoder(Wr, w13s, w2s, sp, max(10, a.steps // 2), a.warmup, a.repeat)
        extra["dense_mlp"] = measure_dense_mlps(sp, 5, 2, 1)

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(shape, w, X, a.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(T / (us_main * 1e-6), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(us_main / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights N(0,0.02), tokens N(0,1))",
        "config": {"workload": shape.name, "T": T, "H": shape.H, "E": shape.E, "k": shape.k, "I": shape.I,
                   "schedule": a.sched, "weight_copies_rotated": R, "active_experts": n_act},
        "us_per_layer": {s: round(v, 2) for s, v in us.items()},
        "us_per_layer_runs": {s: [round(x, 2) for x in v] for s, v in runs.items()},
        "us_per_launch_dist": {s: dist(v) for s, v in per_launch.items()},
        "mfma_frac_whole_layer": round(mfma_frac, 5),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "first_step_warmup_ms": round(warmup_ms, 2),
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
