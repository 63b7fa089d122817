"""GPU parity of the MoE megakernel against the CPU oracle, through the C ABI.

Bar: routing tensors (topk_ids, counts, exp_indptr, perm, slot) bit-exact;
routing weights within 1e-5 relative; layer output within 2e-2 row-wise
relative error (max |got - ref| / max |ref| per token row).  Every schedule
runs the same deterministic task bodies, so the schedules must also agree
with each other bit for bit."""
import numpy as np
import pytest

import oracle
from dynamic_moe_task_amd import workloads as wl
from gpu_util import DeviceLayer, announce, assert_routing_equal, assert_rows_close

pytestmark = pytest.mark.gpu

DYNAMIC_OFF = ("the dynamic push/pop schedule is switched off in the library: its first GPU launch did "
               "not complete (no fault; the test timed out) and the cause is not yet found")
SCHEDS = ["static", pytest.param("dynamic", marks=pytest.mark.skip(reason=DYNAMIC_OFF)), "barrier", "kbk",
          "ordered"]
LIVE = ["static", "barrier", "kbk", "ordered"]


@pytest.fixture(scope="module")
def qwen_weights():
    w = wl.make_weights(wl.DECODE, seed=0)
    return w


@pytest.fixture(scope="module")
def qwen_layer(qwen_weights):
    s = wl.DECODE
    return DeviceLayer((s.H, s.E, s.k, s.I), qwen_weights.Wr, qwen_weights.W13, qwen_weights.Wd, T_max=512)


# ------------------------------------------------------------------ tiny --
@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("sched", SCHEDS)
def test_tiny_layer(sched, norm):
    s = wl.TINY
    w, X = wl.make_layer(s, 0)
    announce(f"tiny T={s.T} sched={sched} norm={norm}")
    ref = oracle.moe(X, w.Wr, w.W13, w.Wd, k=s.k, norm_topk=norm)
    layer = DeviceLayer((s.H, s.E, s.k, s.I), w.Wr, w.W13, w.Wd, T_max=8, norm_topk=norm)
    got = layer.run(X, sched)
    assert_routing_equal(got, ref)
    assert_rows_close(got["out"], ref["out"])


# ---------------------------------------------------------------- decode --
@pytest.fixture(scope="module")
def decode_case(qwen_weights):
    s = wl.DECODE
    rng = np.random.default_rng((0, 16))
    X = wl.to_bf16_bits(rng.standard_normal((s.T, s.H), dtype=np.float32))
    ref = oracle.moe(X, qwen_weights.Wr, qwen_weights.W13, qwen_weights.Wd, k=s.k)
    return X, ref


@pytest.mark.parametrize("sched", SCHEDS)
def test_decode_layer_full_parity(qwen_layer, decode_case, sched):
    X, ref = decode_case
    announce(f"decode T=16 sched={sched}")
    got = qwen_layer.run(X, sched)
    assert_routing_equal(got, ref)
    assert_rows_close(got["out"], ref["out"])


def test_schedules_agree_bit_for_bit(qwen_layer, decode_case):
    X, _ = decode_case
    outs = {}
    for sched in LIVE:
        announce(f"decode T=16 determinism sched={sched}")
        outs[sched] = qwen_layer.run(X, sched)["out"]
    again = qwen_layer.run(X, "static")["out"]
    for sched in LIVE:
        assert np.array_equal(outs[sched], outs["static"]), sched
    assert np.array_equal(again, outs["static"])


@pytest.mark.parametrize("sched", ["static", "ordered",
                                   pytest.param("dynamic", marks=pytest.mark.skip(reason=DYNAMIC_OFF))])
def test_event_invariants(qwen_weights, decode_case, sched):
    # every expert event is notified exactly counts[e] times and completed
    # exactly once when counts[e] > 0; the task counts match the graph
    s = wl.DECODE
    X, ref = decode_case
    layer = DeviceLayer((s.H, s.E, s.k, s.I), qwen_weights.Wr, qwen_weights.W13, qwen_weights.Wd,
                        T_max=64, debug=True)
    announce(f"decode event invariants sched={sched}")
    got = layer.run(X, sched)
    dbg = got["debug"]
    E = s.E
    counts = ref["counts"]
    assert np.array_equal(dbg[:E], counts)
    assert np.array_equal(dbg[E:2 * E], (counts > 0).astype(np.int32))
    info = layer.B.moe_layer_info(layer.desc)
    n_rt = len(oracle.expected_tiles(ref["exp_indptr"], info.bm))
    T = s.T
    expect = [
        -(-T // info.router_tokens) * -(-E // info.router_experts_for(T)),  # R
        -(-T // info.router_tokens),                                 # K
        1,                                                           # S
        -(-T // info.dispatch_tokens) if info.dispatch_tokens else 0,  # D (0: fused into G1's row gather)
        n_rt * (s.I // info.bn1_for(T, s.k)),                        # G1
        n_rt * (s.H // info.bn2_for(T, s.k)),                        # G2
        -(-T // info.combine_tokens),                                # C
    ]
    assert list(dbg[2 * E:2 * E + 7]) == expect
    # C tasks find each of their rows in the row tile that S mapped it to
    assert dbg[2 * E + 7] == T * s.k


@pytest.mark.parametrize("sched", ["static", "barrier", "ordered"])
def test_task_trace(qwen_weights, decode_case, sched):
    # the per-task trace holds one record per task, in per-workgroup slots,
    # with wait <= start <= end-of-body <= end-of-notify in every record
    import torch
    s = wl.DECODE
    X, ref = decode_case
    layer = DeviceLayer((s.H, s.E, s.k, s.I), qwen_weights.Wr, qwen_weights.W13, qwen_weights.Wd, T_max=64)
    B = layer.B
    info = B.moe_layer_info(layer.desc)
    records = info.grid * 64
    tr = torch.zeros(B.trace_words(records), dtype=torch.int32, device="cuda")
    layer.bufs.x[:s.T].copy_(torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).cuda())
    stream = torch.cuda.current_stream().cuda_stream
    announce(f"decode trace sched={sched}")
    B.check(B.moe_layer_launch(layer.desc, s.T, layer.bufs.args(trace=tr), B.SCHEDS[sched], stream))
    B.check(B.etc_sync(stream))
    raw = tr.cpu().numpy().view(np.uint32)
    assert raw[1] == records // info.grid and raw[2] == info.grid
    rec = raw[16:].reshape(-1, 8)
    rec = rec[rec[:, 0] != 0].astype(np.int64)
    typ, wg = rec[:, 0] >> 24, rec[:, 0] & 0xFFFFFF
    n_rt = len(oracle.expected_tiles(ref["exp_indptr"], info.bm))
    T, E = s.T, s.E
    expect = {1: -(-T // info.router_tokens) * -(-E // info.router_experts_for(T)), 2: -(-T // info.router_tokens),
              3: 1, 4: -(-T // info.dispatch_tokens) if info.dispatch_tokens else 0, 5: n_rt * (s.I // info.bn1_for(T, s.k)), 6: n_rt * (s.H // info.bn2_for(T, s.k)),
              7: -(-T // info.combine_tokens)}
    assert {t: int((typ == t).sum()) for t in expect} == expect
    assert wg.max() < info.grid
    # one entry/exit record a workgroup (type 15), every workgroup once
    assert sorted(wg[typ == 15].tolist()) == list(range(info.grid))
    tw = (rec[:, 4] << 32) | rec[:, 3]
    stamps = [tw] + [((rec[:, 4] << 32) | rec[:, j]) for j in (5, 6, 7)]
    stamps = [np.where(t < tw, t + (1 << 32), t) for t in stamps]
    for a, b in zip(stamps, stamps[1:]):
        assert (a <= b).all()


@pytest.mark.parametrize("sched", ["static", "barrier", "ordered"])
def test_watchdog_timeout_is_reported_and_workspace_recovers(qwen_layer, decode_case, sched):
    # a 1 us wait budget makes the first wait that has to poll give up: the
    # launch aborts, every other wait sees the abort, the grid drains, and
    # etc_sync reports ETC_ERR_TIMEOUT.  The next launch on the same workspace
    # (counter sets reset by the epoch, also after an abort) is correct.
    X, ref = decode_case
    B = qwen_layer.B
    announce(f"decode watchdog 1us sched={sched}")
    got = qwen_layer.run(X, sched, watchdog_us=1, check_status=False)
    assert got["rc"] == B.ETC_ERR_TIMEOUT
    announce(f"decode after watchdog sched={sched}")
    again = qwen_layer.run(X, sched)
    assert_routing_equal(again, ref)
    assert_rows_close(again["out"], ref["out"])


# --------------------------------------------------------------- prefill --
def _sample_tokens(ids, T, n_each=16):
    # first and last tokens, and tokens of the most loaded expert
    hot = np.bincount(ids.reshape(-1)).argmax()
    hot_tokens = np.nonzero((ids == hot).any(axis=1))[0]
    rng = np.random.default_rng(T)
    pick = (list(range(n_each)) + list(range(T - n_each, T)) + list(hot_tokens[:n_each])
            + list(rng.choice(T, size=min(T, n_each), replace=False)))
    return np.array(sorted(set(int(t) for t in pick)), np.int32)


@pytest.fixture(scope="module")
def prefill_case(qwen_weights):
    s = wl.PREFILL_ZIPF
    w, X = wl.make_layer(s, 0)
    assert np.array_equal(w.Wr, qwen_weights.Wr)  # same seed, same weights
    layer = DeviceLayer((s.H, s.E, s.k, s.I), qwen_weights.Wr, qwen_weights.W13, qwen_weights.Wd,
                        T_max=256, bias=w.bias)
    ref = oracle.route(X, qwen_weights.Wr, s.k, bias=w.bias)
    # every output row of the batch (the oracle's rows, once for all schedules)
    ref["out"] = oracle.moe_tokens(np.arange(s.T, dtype=np.int32), X, qwen_weights.W13, qwen_weights.Wd,
                                   ref["topk_ids"], ref["topk_w"])
    return layer, X, ref


@pytest.mark.parametrize("sched", SCHEDS)
def test_prefill_zipf_full_parity(prefill_case, sched):
    layer, X, ref = prefill_case
    announce(f"prefill zipf T=256 sched={sched}")
    got = layer.run(X, sched)
    assert_routing_equal(got, ref)
    assert (ref["counts"] == 0).sum() > 0 and ref["counts"].max() > 64  # skewed, as the workload intends
    assert_rows_close(got["out"], ref["out"])


# ----------------------------------------------------------------- sweep --
def test_batch_sweep_one_template(qwen_layer, qwen_weights):
    # one compiled kernel, one workspace, T changes per launch; every output
    # row is checked on every 10th step of the seeded 200-step sweep and on
    # its smallest and largest batch, routing on every step
    s = wl.SWEEP
    Bs = wl.sweep_batches(0)
    full = set(list(range(0, len(Bs), 10)) + [int(np.argmin(Bs)), int(np.argmax(Bs))])
    extra = [(1000, 1), (1001, 512), (1002, 33)]
    cases = [(st, int(Bs[st])) for st in range(len(Bs))] + extra
    for i, (step, T) in enumerate(cases):
        sched = LIVE[i % len(LIVE)]
        X = wl.sweep_tokens(s, step, T, seed=0)
        announce(f"sweep step={step} T={T} sched={sched}")
        got = qwen_layer.run(X, sched)
        ref = oracle.route(X, qwen_weights.Wr, s.k)
        assert_routing_equal(got, ref)
        tok = (np.arange(T, dtype=np.int32) if (step in full or step >= 1000)
               else np.unique(np.array([0, T // 2, T - 1], np.int32)))
        rows = oracle.moe_tokens(tok, X, qwen_weights.W13, qwen_weights.Wd, ref["topk_ids"], ref["topk_w"])
        assert_rows_close(got["out"][tok], rows)


# ------------------------------------------------- the pages' token counts --
@pytest.fixture(scope="module")
def large_layer(qwen_weights):
    s = wl.DECODE
    return DeviceLayer((s.H, s.E, s.k, s.I), qwen_weights.Wr, qwen_weights.W13, qwen_weights.Wd, T_max=4096)


@pytest.mark.parametrize("T", [1024, 4096])
@pytest.mark.parametrize("sched", SCHEDS)
def test_qwen_shape_large_batches(large_layer, qwen_weights, T, sched):
    # the token counts of the pages' MoE-layer table beyond decode: routing
    # bit-exact, and sampled rows (the first and last tokens, tokens of the
    # most loaded expert, random tokens) against the oracle
    s = wl.DECODE
    X = wl.sweep_tokens(s, 7000 + T, T, seed=0)
    ref = oracle.route(X, qwen_weights.Wr, s.k)
    announce(f"qwen T={T} sched={sched}")
    got = large_layer.run(X, sched)
    assert_routing_equal(got, ref)
    tok = _sample_tokens(ref["topk_ids"], T)
    assert len(tok) >= 48
    rows = oracle.moe_tokens(tok, X, qwen_weights.W13, qwen_weights.Wd, ref["topk_ids"], ref["topk_w"])
    assert_rows_close(got["out"][tok], rows)


# ------------------------------------------------------------ edge shapes --
EDGE = [
    # (T, H, E, k, I, norm, bias, T_max)
    (1, 128, 8, 2, 256, True, False, 1),       # single token, T == T_max
    (5, 256, 16, 4, 128, True, True, 9),       # ragged tiles, with bias
    (37, 128, 8, 8, 256, True, False, 40),     # k == E: every expert gets every token
    (3, 128, 1, 1, 128, True, False, 4),       # one expert: dense MLP
    (64, 384, 256, 16, 128, False, False, 64), # E = 256, k = 16, plain softmax weights
    (2, 640, 64, 6, 384, True, False, 2),      # most experts get no token
    (4096, 128, 64, 8, 128, True, False, 4096),  # T == T_max == 4096: eight scan chunks
    (700, 128, 16, 4, 128, True, True, 800),   # two scan chunks, the second ragged
    (16384, 128, 8, 2, 128, True, False, 16384),  # largest T_max: 32 scan chunks, 8 experts
    (8, 16384, 8, 2, 128, True, False, 8),     # hidden size 16384
    (8, 128, 8, 2, 16384, True, False, 8),     # expert intermediate size 16384
    (8, 40960, 8, 2, 128, True, False, 8),     # largest hidden size
    (2, 256, 1, 1, 40960, True, False, 2),     # one expert of the largest intermediate size
    (512, 128, 16, 8, 128, True, False, 512),  # T * k = 4096: the largest batch with the routing tables in LDS
    (300, 128, 32, 14, 128, True, False, 320), # T * k = 4200: one scan chunk, routing tables in memory
    (12, 128, 64, 8, 256, True, False, 16),    # between one and two G tiles per workgroup of the grid
    (256, 384, 32, 8, 640, True, True, 256),   # column-split G tiles over 3 (G1) and 5 (G2) staged chunks
    (300, 256, 16, 8, 384, True, False, 320),  # column-split G tiles, 2 (G1) and 3 (G2) chunks, T < T_max
    (2048, 2048, 64, 4, 128, True, False, 2048),  # 32-expert router tiles, unpredicated (H a multiple of 1024);
                                                  # two C tasks a workgroup, two row chunks a thread in each
    (2050, 128, 44, 4, 128, True, True, 2304),  # 32-expert router tiles: a 2-token tile, a 12-expert tile
]


_EDGE_CACHE = {}


def _edge_inputs(case):
    # inputs and the oracle's result, computed once per case for all schedules
    # (a few hundred MB at most over all cases)
    if case not in _EDGE_CACHE:
        T, H, E, k, I, norm, has_bias, T_max = case
        rng = np.random.default_rng(T * 7919 + E)
        Wr = wl.to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.05))
        W13 = wl.to_bf16_bits(rng.standard_normal((E, 2 * I, H), dtype=np.float32) * np.float32(0.05))
        Wd = wl.to_bf16_bits(rng.standard_normal((E, H, I), dtype=np.float32) * np.float32(0.05))
        X = wl.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
        bias = (rng.standard_normal(E) * 0.5).astype(np.float32) if has_bias else None
        ref = oracle.moe(X, Wr, W13, Wd, k=k, norm_topk=norm, bias=bias)
        _EDGE_CACHE[case] = (Wr, W13, Wd, X, bias, ref)
    return _EDGE_CACHE[case]


@pytest.mark.parametrize("case", EDGE, ids=[f"T{c[0]}H{c[1]}E{c[2]}k{c[3]}I{c[4]}" for c in EDGE])
@pytest.mark.parametrize("sched", ["static", pytest.param("dynamic", marks=pytest.mark.skip(reason=DYNAMIC_OFF)),
                                   "kbk", "barrier", "ordered"])
def test_edge_shapes(case, sched):
    T, H, E, k, I, norm, has_bias, T_max = case
    Wr, W13, Wd, X, bias, ref = _edge_inputs(case)
    announce(f"edge {case} sched={sched}")
    layer = DeviceLayer((H, E, k, I), Wr, W13, Wd, T_max=T_max, bias=bias, norm_topk=norm)
    got = layer.run(X, sched)
    assert_routing_equal(got, ref)
    assert_rows_close(got["out"], ref["out"])


def test_repeated_launches_reuse_workspace(qwen_layer, qwen_weights):
    # the counter sets are reset by the kernels themselves: alternate
    # schedules and sizes on one workspace, every launch must still match
    s = wl.DECODE
    for i, (T, sched) in enumerate([(16, "static"), (3, "barrier"), (16, "kbk"), (40, "static"),
                                    (1, "barrier"), (7, "static"), (7, "kbk"), (16, "kbk"),
                                    (9, "static"), (2, "barrier"), (33, "ordered"), (1, "ordered"),
                                    (16, "ordered"), (5, "static")]):
        X = wl.sweep_tokens(s, 5000 + i, T, seed=0)
        announce(f"repeat i={i} T={T} sched={sched}")
        got = qwen_layer.run(X, sched)
        ref = oracle.route(X, qwen_weights.Wr, s.k)
        assert_routing_equal(got, ref)
        tok = np.unique(np.array([0, T - 1], np.int32))
        rows = oracle.moe_tokens(tok, X, qwen_weights.W13, qwen_weights.Wd, ref["topk_ids"], ref["topk_w"])
        assert_rows_close(got["out"][tok], rows)
