"""CPU pins of the oracle against things other than itself: hand-derived
values, closed forms, brute force on tiny inputs, library routines on special
cases, and invariants.  No GPU, no HIP library."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from dynamic_moe_task_amd import workloads as wl

F32 = np.float32


def bits(x):
    """float32 value(s) -> bf16 bits via torch's own conversion (RNE)."""
    t = torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def from_bits(b):
    return oracle.bf16_bits_to_f64(b)


# ---------------------------------------------------------------- bf16 RNE --
@pytest.mark.parametrize("value,expect", [
    (1.0, 0x3F80),
    (-2.0, 0xC000),
    (1.0 + 2.0 ** -8, 0x3F80),               # exact tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),           # exact tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (3.0e38, 0x7F62),
])
def test_bf16_rne_hand_values(value, expect):
    assert oracle.f32_to_bf16_bits(value) == expect


def test_bf16_rne_matches_torch_on_random_and_ties():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000).astype(F32) * F32(37.0)
    u = v.view(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    allv = np.concatenate([v, ties])
    mine = np.array([oracle.f32_to_bf16_bits(float(x)) for x in allv], np.uint16)
    assert np.array_equal(mine, bits(allv))
    # the input generator's vectorised rounding agrees with torch as well
    assert np.array_equal(wl.to_bf16_bits(allv), bits(allv))


# ---------------------------------------------------- router logit contract --
def _one_row(H, xs, ws):
    X = np.zeros((1, H), np.uint16)
    W = np.zeros((1, H), np.uint16)
    for h, v in xs.items():
        X[0, h] = bits(v)
    for h, v in ws.items():
        W[0, h] = bits(v)
    return X, W


def test_logit_tree_order_hand_value():
    # H = 512: 64 chunks, chunk c on lane c.  Lane 0 holds 2^24, lanes 1..63
    # hold 1.  Halving tree: 2^24+1 ties to 2^24, then +2, +4, +8, +16, +32
    # are exact: 2^24 + 62.  A sequential sum would give 2^24, fp64 2^24+63.
    H = 512
    X, W = _one_row(H, {8 * l: 1.0 for l in range(64)},
                    {0: 2.0 ** 24, **{8 * l: 1.0 for l in range(1, 64)}})
    L = oracle.router_logits(X, W)
    assert L[0, 0] == F32(2.0 ** 24 + 62)
    assert oracle.router_logits_f64(X, W)[0, 0] == 2.0 ** 24 + 63


def test_logit_lane_order_hand_value():
    # H = 1024: lane 0 owns chunks 0 and 64 (h = 0..7 and 512..519).  Its
    # elements go in ascending h: 1 + 1 = 2, then 2 + 2^24 is exact.  The
    # reverse order would lose both ones (2^24 + 1 ties to 2^24).
    H = 1024
    X, W = _one_row(H, {0: 1.0, 1: 1.0, 512: 1.0}, {0: 1.0, 1: 1.0, 512: 2.0 ** 24})
    assert oracle.router_logits(X, W)[0, 0] == F32(2.0 ** 24 + 2)


def test_logit_bias_added_last():
    X, W = _one_row(512, {0: 1.0}, {0: 0.5})
    b = np.array([0.25], np.float32)
    assert oracle.router_logits(X, W, b)[0, 0] == F32(0.75)


def test_logits_close_to_fp64_and_onehot_exact():
    shape = wl.TINY
    w, X = wl.make_layer(shape, 0)
    L32 = oracle.router_logits(X, w.Wr)
    L64 = oracle.router_logits_f64(X, w.Wr)
    absprod = np.abs(from_bits(X)) @ np.abs(from_bits(w.Wr)).T
    assert np.all(np.abs(L32 - L64) <= 64 * 2.0 ** -24 * absprod + 1e-30)
    # one-hot activations select a single weight exactly
    Xo = np.zeros((3, shape.H), np.uint16)
    for t, h in enumerate([0, 77, 127]):
        Xo[t, h] = bits(1.0)
    Lo = oracle.router_logits(Xo, w.Wr)
    for t, h in enumerate([0, 77, 127]):
        assert np.array_equal(Lo[t], from_bits(w.Wr[:, h]).astype(np.float32))


# ------------------------------------------------------------------- top-k --
def _brute_topk(row, k):
    # every k-subset, each listed in its own best-first order; the winner is
    # the lexicographically greatest sequence of (value, -index) keys
    best = None
    for sub in itertools.combinations(range(len(row)), k):
        seq = sorted(sub, key=lambda e: (-row[e], e))
        key = [(row[e], -e) for e in seq]
        if best is None or key > best[0]:
            best = (key, seq)
    return best[1]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(2, 9))
    k = int(rng.integers(1, E + 1))
    T = 7
    # few distinct values so that ties are frequent
    L = rng.integers(-2, 3, size=(T, E)).astype(np.float32) * F32(0.5)
    ids, w = oracle.topk(L, k, norm_topk=True)
    for t in range(T):
        assert list(ids[t]) == _brute_topk(list(L[t]), k)


def test_topk_weights_two_formulas():
    rng = np.random.default_rng(7)
    L = (rng.standard_normal((5, 10)) * 2).astype(np.float32)
    k = 3
    ids, w = oracle.topk(L, k, norm_topk=True)
    _, wfull = oracle.topk(L, k, norm_topk=False)
    # softmax over all E, then renormalise over the chosen k
    p = np.exp(L.astype(np.float64) - L.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-6)
    np.testing.assert_allclose(wfull, sel, rtol=1e-6)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_topk_rejects_nan():
    L = np.zeros((1, 4), np.float32)
    L[0, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.topk(L, 2)


# ---------------------------------------------- counts / indptr / permutation --
def _check_routing_invariants(ids, E, counts, indptr, perm, slot):
    T, k = ids.shape
    flat = ids.reshape(-1)
    assert counts.sum() == T * k
    assert indptr[0] == 0 and indptr[-1] == T * k
    assert np.all(np.diff(indptr) == counts) and np.all(np.diff(indptr) >= 0)
    assert sorted(perm.tolist()) == list(range(T * k))
    assert np.array_equal(slot[perm], np.arange(T * k))
    for e in range(E):
        seg = perm[indptr[e]:indptr[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)  # stable: ascending flat index
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (4, 8, 2), (37, 16, 4), (64, 128, 8), (3, 5, 5)])
def test_route_scan_invariants_and_stable_sort(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, indptr, perm, slot = oracle.route_scan(ids, E)
    _check_routing_invariants(ids, E, counts, indptr, perm, slot)
    # a library stable sort of the flat expert ids gives the same permutation
    assert np.array_equal(perm, np.argsort(ids.reshape(-1), kind="stable"))


def test_tiny_layer_routing_invariants():
    w, X = wl.make_layer(wl.TINY, 0)
    r = oracle.route(X, w.Wr, wl.TINY.k)
    _check_routing_invariants(r["topk_ids"], wl.TINY.E, r["counts"], r["exp_indptr"],
                              r["perm"], r["slot"])


# ----------------------------------------------------- expert maths pins --
def _dense_swiglu_ref(X, Wg, Wu, Wd):
    """Dense SwiGLU MLP with the same rounding points, in torch fp64."""
    x = torch.from_numpy(from_bits(X))
    g = x @ torch.from_numpy(from_bits(Wg)).T
    u = x @ torch.from_numpy(from_bits(Wu)).T
    h = (g * torch.sigmoid(g) * u).float().to(torch.bfloat16).double()
    y = (h @ torch.from_numpy(from_bits(Wd)).T).float().to(torch.bfloat16)
    return y.view(torch.int16).numpy().view(np.uint16)


def _ulp_close(a_bits, b_bits, ulps=1):
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    # same sign and within `ulps` of each other in the bf16 ordering
    sa = np.where(a & 0x8000, -(a & 0x7FFF), a & 0x7FFF)
    sb = np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(sa - sb) <= ulps


def test_single_expert_is_dense_mlp():
    # E = 1, k = 1: routing weight is exactly 1, so out = Y = dense MLP(X).
    rng = np.random.default_rng(3)
    T, H, I = 9, 64, 128
    X = wl.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    Wr = wl.to_bf16_bits(rng.standard_normal((1, H), dtype=np.float32) * F32(0.02))
    W13 = wl.to_bf16_bits(rng.standard_normal((1, 2 * I, H), dtype=np.float32) * F32(0.1))
    Wd = wl.to_bf16_bits(rng.standard_normal((1, H, I), dtype=np.float32) * F32(0.1))
    r = oracle.moe(X, Wr, W13, Wd, k=1)
    assert np.all(r["topk_w"] == 1.0)
    ref = _dense_swiglu_ref(X, W13[0, :I], W13[0, I:], Wd[0])
    assert np.mean(_ulp_close(r["out"], ref, 0)) > 0.99
    assert np.all(_ulp_close(r["out"], ref, 1))


def test_identical_experts_equal_dense_mlp():
    # Every expert the same and norm_topk: out = bf16(sum_j w_j * Y) with
    # sum_j w_j = 1, i.e. the dense MLP up to one final rounding.
    rng = np.random.default_rng(4)
    T, H, I, E, k = 6, 64, 64, 8, 3
    X = wl.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    Wr = wl.to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * F32(0.3))
    one13 = wl.to_bf16_bits(rng.standard_normal((2 * I, H), dtype=np.float32) * F32(0.1))
    oned = wl.to_bf16_bits(rng.standard_normal((H, I), dtype=np.float32) * F32(0.1))
    W13 = np.broadcast_to(one13, (E, 2 * I, H)).copy()
    Wd = np.broadcast_to(oned, (E, H, I)).copy()
    r = oracle.moe(X, Wr, W13, Wd, k=k)
    ref = _dense_swiglu_ref(X, one13[:I], one13[I:], oned)
    assert np.all(_ulp_close(r["out"], ref, 1))


def test_scalar_permutation_experts_closed_form():
    # Expert e: gate = a_e P_e x, up = b_e Q_e x, down = c_e R_e h with
    # permutation matrices, so every output element has a closed form.  A
    # transposed weight layout, swapped gate/up halves or a wrong expert
    # index all change the answer.
    rng = np.random.default_rng(5)
    T, H, E, k = 5, 64, 4, 2
    I = H
    a = [0.5, 1.0, 2.0, -1.5]
    b = [1.25, -0.75, 0.5, 2.0]
    c = [1.0, 0.5, -2.0, 0.25]
    P = [rng.permutation(H) for _ in range(E)]
    Q = [rng.permutation(H) for _ in range(E)]
    R = [rng.permutation(H) for _ in range(E)]
    W13 = np.zeros((E, 2 * I, H), np.uint16)
    Wd = np.zeros((E, H, I), np.uint16)
    for e in range(E):
        W13[e, np.arange(I), P[e]] = bits(a[e])
        W13[e, I + np.arange(I), Q[e]] = bits(b[e])
        Wd[e, np.arange(H), R[e]] = bits(c[e])
    X = wl.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    Wr = wl.to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32))
    r = oracle.moe(X, Wr, W13, Wd, k=k, intermediates=True)
    x = from_bits(X)
    expect = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = r["topk_ids"][t, j]
            g = a[e] * x[t, P[e]]
            u = b[e] * x[t, Q[e]]
            h = from_bits(wl.to_bf16_bits((g / (1 + np.exp(-g)) * u).astype(np.float32)))
            y = from_bits(wl.to_bf16_bits((c[e] * h[R[e]]).astype(np.float32)))
            expect[t] += float(r["topk_w"][t, j]) * y
    ebits = wl.to_bf16_bits(expect.astype(np.float32))
    assert np.all(_ulp_close(r["out"], ebits, 0))


def test_moe_tokens_matches_full_layer():
    w, X = wl.make_layer(wl.TINY, 0)
    r = oracle.moe(X, w.Wr, w.W13, w.Wd, k=wl.TINY.k)
    rows = oracle.moe_tokens([3, 0, 2], X, w.W13, w.Wd, r["topk_ids"], r["topk_w"])
    assert np.array_equal(rows, r["out"][[3, 0, 2]])


def test_tiny_layer_against_fp64_unrounded():
    # The oracle rounds Hmid and Y to bf16; an fp64 version with no
    # intermediate rounding stays within the output tolerance.
    shape = wl.TINY
    w, X = wl.make_layer(shape, 0)
    r = oracle.moe(X, w.Wr, w.W13, w.Wd, k=shape.k)
    x = from_bits(X)
    W13 = from_bits(w.W13)
    Wd = from_bits(w.Wd)
    ref = np.zeros((shape.T, shape.H))
    for t in range(shape.T):
        for j in range(shape.k):
            e = r["topk_ids"][t, j]
            g = W13[e, :shape.I] @ x[t]
            u = W13[e, shape.I:] @ x[t]
            ref[t] += r["topk_w"][t, j] * (Wd[e] @ (g / (1 + np.exp(-g)) * u))
    got = from_bits(r["out"])
    err = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert np.all(err < 2e-2)


# --------------------------------------------------------------- split-K --
def _golden(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    kv = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if " = " in line:
            k_, v_ = line.split(" = ", 1)
            kv[k_.strip()] = v_.strip()
        elif "->" in line:
            k_, v_ = line.split("->", 1)
            kv[k_.strip()] = v_.strip()
    return kv


def test_splitk_closed_form():
    g = _golden("fig3_splitk_wiring.txt")
    nsplit = int(g["wait_count"])
    assert nsplit == 4
    rng = np.random.default_rng(9)
    n, bk = 50, 16
    A = rng.integers(-1000, 1000, size=(n, nsplit * bk)).astype(np.int32)
    B, C, notif = oracle.splitk(A, nsplit)
    assert np.array_equal(C, A.sum(axis=1))
    assert np.array_equal(B, A.reshape(n, nsplit, bk).sum(axis=2))
    assert np.all(notif == nsplit)


# ---------------------------------------------------------- event model --
from oracle import events as ev  # noqa: E402


def test_fig4_instantiation_shapes():
    g = _golden("fig4_instantiation.txt")
    t = ev.ETensor(["B", 2], wait_count=1)
    assert t.instantiate(B=1) == tuple(int(v) for v in g["B=1"].split(","))
    assert t.instantiate(B=2) == tuple(int(v) for v in g["B=2"].split(","))


def test_rs_walkthrough_counter():
    g = _golden("rs_walkthrough.txt")
    st = ev.EventState()
    st.declare("rs", (1,), int(g["initial"]))
    key = ("rs", (0,))
    assert st.remaining[key] == 2 and not st.ready(key)
    st.notify(key)
    assert st.remaining[key] == int(g["after_notify_1"].split()[0]) and not st.ready(key)
    st.notify(key)
    assert st.remaining[key] == 0 and st.ready(key) and st.fired[key] == 1
    st.notify(key)
    assert st.errors  # a third notify is an over-notification


def test_edge_maps():
    assert ev.edge_apply("ij->i", (3, 2)) == (3,)
    assert ev.edge_apply("i->i", (5,)) == (5,)
    with pytest.raises(ValueError):
        ev.parse_edge("i->j")


def _splitk_graph(A, nsplit):
    n = A.shape[0]
    bk = A.shape[1] // nsplit
    g = _golden("fig3_splitk_wiring.txt")
    B = np.zeros((n, nsplit), np.int64)
    C = np.zeros(n, np.int64)
    st = ev.EventState()
    st.declare("ev", (n,), nsplit)
    tasks = []
    for i in range(n):
        for j in range(nsplit):
            def run(i=i, j=j):
                B[i, j] = A[i, j * bk:(j + 1) * bk].sum()
            tasks.append(ev.Task("partial_sum", (i, j), [],
                                 [("ev", ev.edge_apply(g["out_edge"], (i, j)))], run))
    for i in range(n):
        def run(i=i):
            C[i] = B[i].sum()
        tasks.append(ev.Task("final_sum", (i,), [("ev", ev.edge_apply(g["in_edge"], (i,)))], [], run))
    return tasks, st, B, C


@pytest.mark.parametrize("seed", range(4))
def test_splitk_through_event_model(seed):
    rng = np.random.default_rng(seed)
    n, nsplit, bk = 6, 4, 8
    A = rng.integers(-50, 50, size=(n, nsplit * bk))
    # dynamic schedule, random pop order
    tasks, st, B, C = _splitk_graph(A, nsplit)
    ev.run_dynamic(tasks, st, seed=seed)
    assert np.array_equal(C, A.sum(axis=1)) and not st.errors
    assert all(v == 1 for v in st.fired.values())
    # static schedule: 3 workers, phase-ordered round-robin lists
    tasks, st, B, C = _splitk_graph(A, nsplit)
    W = 3
    lists = [[i for i in range(len(tasks)) if i % W == w] for w in range(W)]
    ev.run_static(tasks, st, W, lists)
    assert np.array_equal(C, A.sum(axis=1)) and not st.errors


def test_static_schedule_not_phase_ordered_deadlocks():
    # A worker list that puts a waiter before the producer it waits on, on
    # the same worker, can never progress: the model reports it.
    A = np.ones((1, 8), np.int64)
    tasks, st, B, C = _splitk_graph(A, 4)
    lists = [[4, 0, 1, 2, 3]]
    with pytest.raises(RuntimeError):
        ev.run_static(tasks, st, 1, lists)


def test_moe_event_graph_counts_and_single_fire():
    # Data-dependent update: expert e's counter starts at counts[e]; each
    # routed (t, j) notifies ids[t, j]; the expert's tiles over
    # [exp_indptr[e], exp_indptr[e+1]) wait on it.  Every event fires once.
    w, X = wl.make_layer(wl.TINY, 0)
    r = oracle.route(X, w.Wr, wl.TINY.k)
    E = wl.TINY.E
    counts = r["counts"]
    st = ev.EventState()
    st.declare("exp", (E,), lambda idx: int(counts[idx[0]]))
    tasks = []
    ids = r["topk_ids"]
    for t in range(ids.shape[0]):
        tasks.append(ev.Task("dispatch", (t,), [], [("exp", (int(e),)) for e in ids[t]]))
    bm = 2
    for (e, lo, hi) in oracle.expected_tiles(r["exp_indptr"], bm):
        tasks.append(ev.Task("g1", (e, lo), [("exp", (e,))], []))
    ev.run_dynamic(tasks, st, seed=1)
    for e in range(E):
        assert st.notified[("exp", (e,))] == counts[e]
        assert st.fired[("exp", (e,))] == 1
    n_tiles = sum(math.ceil(c / bm) for c in counts)
    assert len(oracle.expected_tiles(r["exp_indptr"], bm)) == n_tiles


def _moe_layer_graph(T, E, k, bm, n1, n2, seed):
    """Event graph of one MoE layer as the megakernel runs it: R(tt, et) ->
    ev_logit[tt] -> K(tt) -> (ev_exp[e] once per routed pair, ev_route) ->
    S -> ev_scan -> G1(rt, n) -> ev_h[rt] -> G2(rt, n) -> ev_y[rt] -> C(ct),
    where C waits on every row tile holding one of its tokens' rows.  Row
    tiles are cut from exp_indptr as the oracle defines them."""
    rng = np.random.default_rng(seed)
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int64)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    indptr = np.concatenate([[0], np.cumsum(counts)])
    tiles = oracle.expected_tiles(indptr, bm)
    row_tile = {}
    for rt, (e, lo, hi) in enumerate(tiles):
        for r in range(lo, hi):
            row_tile[r] = rt
    rank = {}
    slot = np.zeros((T, k), np.int64)
    for t in range(T):  # stable: rows of one expert in ascending token order
        for j in range(k):
            e = int(ids[t, j])
            slot[t, j] = indptr[e] + rank.get(e, 0)
            rank[e] = rank.get(e, 0) + 1
    rt_tok, et_exp, ct_tok = 4, 4, 2
    ntt, net, nct = -(-T // rt_tok), -(-E // et_exp), -(-T // ct_tok)
    st = ev.EventState()
    st.declare("logit", (ntt,), net)
    st.declare("route", (1,), ntt)
    st.declare("exp", (E,), lambda i: int(counts[i[0]]))
    st.declare("scan", (1,), 1)
    st.declare("h", (len(tiles),), n1)
    st.declare("y", (len(tiles),), n2)
    tasks, ph = [], {n: [] for n in ("R", "K", "S", "G1", "G2", "C")}

    def add(name, key, waits, notifies):
        ph[name].append(len(tasks))
        tasks.append(ev.Task(name, key, waits, notifies))

    for tt in range(ntt):
        for et in range(net):
            add("R", (tt, et), [], [("logit", (tt,))])
    for tt in range(ntt):
        pairs = [("exp", (int(ids[t, j]),)) for t in range(tt * rt_tok, min(T, tt * rt_tok + rt_tok))
                 for j in range(k)]
        add("K", (tt,), [("logit", (tt,))], pairs + [("route", (0,))])
    add("S", (0,), [("route", (0,))], [("scan", (0,))])
    for rt, (e, lo, hi) in enumerate(tiles):
        for n in range(n1):
            add("G1", (rt, n), [("scan", (0,)), ("exp", (e,))], [("h", (rt,))])
    for rt in range(len(tiles)):
        for n in range(n2):
            add("G2", (rt, n), [("h", (rt,))], [("y", (rt,))])
    for ct in range(nct):
        rts = sorted({row_tile[int(slot[t, j])] for t in range(ct * ct_tok, min(T, ct * ct_tok + ct_tok))
                      for j in range(k)})
        add("C", (ct,), [("scan", (0,))] + [("y", (rt,)) for rt in rts], [])
    return tasks, st, ph


@pytest.mark.parametrize("workers", [5, 8, 16])
@pytest.mark.parametrize("seed", range(3))
def test_ordered_claims_complete_the_moe_graph(workers, seed):
    # The ORDERED schedule: R, K, S dealt in phase order, then one stream
    # of G1 tiles followed by G2 tiles claimed in index order from per-group
    # counters three ahead, then C dealt.  With workers of random speed every
    # task completes and every non-empty event fires exactly once.
    tasks, st, ph = _moe_layer_graph(T=12, E=8, k=2, bm=4, n1=3, n2=2, seed=seed)
    phases = [("deal", ph["R"]), ("deal", ph["K"]), ("deal", ph["S"]), ("claim", ph["G1"] + ph["G2"]),
              ("deal", ph["C"])]
    order = ev.run_ordered(tasks, st, workers, phases, groups=4, seed=seed)
    assert sorted(order) == list(range(len(tasks))) and not st.errors
    assert all(v == 1 for v in st.fired.values())


@pytest.mark.parametrize("workers", [3, 8, 16, 40])
@pytest.mark.parametrize("seed", range(3))
def test_ordered_small_batch_runner_completes_the_moe_graph(workers, seed):
    # The small-batch form: one counter for all workers, each worker's first
    # two G tiles dealt (w, workers + w; the worker that ran S and worker
    # workers - 1 swap theirs), then one claim per finished tile, two tiles
    # held.  With fewer tiles than two per worker (40 workers) some workers
    # get one dealt tile or none and claim nothing.
    tasks, st, ph = _moe_layer_graph(T=12, E=8, k=2, bm=4, n1=3, n2=2, seed=seed)
    phases = [("deal", ph["R"]), ("deal", ph["K"]), ("deal", ph["S"]), ("claim", ph["G1"] + ph["G2"]),
              ("deal", ph["C"])]
    s_worker = (len(ph["R"]) + len(ph["K"])) % workers
    order = ev.run_ordered(tasks, st, workers, phases, groups=1, ahead=2, dealt=2, seed=seed, swap=s_worker)
    assert sorted(order) == list(range(len(tasks))) and not st.errors
    assert all(v == 1 for v in st.fired.values())


def test_ordered_claims_out_of_graph_order_deadlock():
    # Claiming G2 tiles before G1 tiles breaks the argument: every worker
    # then holds a G2 tile whose G1 producers nobody can start.
    tasks, st, ph = _moe_layer_graph(T=12, E=8, k=2, bm=4, n1=3, n2=2, seed=0)
    phases = [("deal", ph["R"]), ("deal", ph["K"]), ("deal", ph["S"]), ("claim", ph["G2"] + ph["G1"]),
              ("deal", ph["C"])]
    with pytest.raises(RuntimeError):
        ev.run_ordered(tasks, st, 4, phases, groups=4, seed=0)


# ===================================================== decoder-layer oracle --
# Pins of the decoder layer's steps (RMSNorm, projection, rotary embedding,
# decode attention, the whole layer) against closed forms, special cases and
# values worked out by hand, none of which retypes the oracle's formula.
def _bits(a):
    return wl.to_bf16_bits(np.asarray(a, np.float32))


def _f(b):
    return oracle.bf16_bits_to_f64(np.asarray(b, np.uint16))


def test_rmsnorm_hand_values_and_weight():
    # x = (3, 4): mean square 12.5, so y = x / sqrt(12.5) * g
    y = oracle.rmsnorm(_bits([[3.0, 4.0]]), _bits([1.0, 2.0]), eps=0.0)
    np.testing.assert_allclose(_f(y)[0], [3 / np.sqrt(12.5), 2 * 4 / np.sqrt(12.5)], rtol=4e-3)
    # a constant row normalises to the sign of the constant, whatever its size
    for c in (-7.5, 0.015625, 1000.0):
        y = oracle.rmsnorm(_bits(np.full((1, 64), c)), _bits(np.ones(64)), eps=0.0)
        assert np.all(_f(y) == np.sign(c))
    # eps enters under the square root: x = 0 stays 0, and a tiny x is damped
    y = oracle.rmsnorm(_bits(np.full((1, 8), 1e-3)), _bits(np.ones(8)), eps=1.0)
    np.testing.assert_allclose(_f(y), 1e-3 / np.sqrt(1e-6 + 1.0), rtol=4e-3)


def test_linear_identity_and_column_pick():
    rng = np.random.default_rng(3)
    x = _bits(rng.standard_normal((5, 16)))
    eye = _bits(np.eye(16))
    assert np.array_equal(oracle.linear(x, eye), x)  # W = I returns x exactly
    pick = np.zeros((3, 16), np.float32)
    pick[0, 7] = pick[1, 0] = pick[2, 15] = 1.0       # row n of W selects one input column
    y = oracle.linear(x, _bits(pick))
    assert np.array_equal(y, x[:, [7, 0, 15]])        # a transposed W would fail here


def test_rope_hand_values():
    # d = 4, theta = 10000: frequencies 1 and 1/100; pairs (0, 2) and (1, 3)
    v = _bits([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0], [0.0, 0.0, 1.0, 0.0]])
    r = _f(oracle.rope(v, pos=1.0, theta=10000.0))
    c, s = np.cos(1.0), np.sin(1.0)
    c2, s2 = np.cos(0.01), np.sin(0.01)
    np.testing.assert_allclose(r[0], [c, 0, s, 0], atol=4e-3)
    np.testing.assert_allclose(r[1], [0, c2, 0, s2], atol=4e-3)
    np.testing.assert_allclose(r[2], [-s, 0, c, 0], atol=4e-3)


def test_rope_is_a_rotation():
    rng = np.random.default_rng(4)
    v = _bits(rng.standard_normal((6, 128)))
    assert np.array_equal(oracle.rope(v, 0.0, 1e6), v)  # position 0: identity
    r = _f(oracle.rope(v, 4096.0, 1e6))
    x = _f(v)
    # every (i, i + 64) pair keeps its length
    n0 = x[:, :64] ** 2 + x[:, 64:] ** 2
    n1 = r[:, :64] ** 2 + r[:, 64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=2e-2, atol=1e-3)
    # and the rotation of pair i by angle a: the dot product of two rotated
    # vectors depends only on the difference of their positions
    q, kv = _bits(rng.standard_normal((1, 128))), _bits(rng.standard_normal((1, 128)))
    d1 = (_f(oracle.rope(q, 100.0, 1e6)) * _f(oracle.rope(kv, 90.0, 1e6))).sum()
    d2 = (_f(oracle.rope(q, 10.0, 1e6)) * _f(oracle.rope(kv, 0.0, 1e6))).sum()
    assert abs(d1 - d2) < 0.05 * (abs(d2) + 1.0)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    nq, nkv, d, L = 4, 2, 16, 9
    q = _bits(rng.standard_normal((nq, d)))
    V = rng.standard_normal((nkv, L, d)).astype(np.float32)
    # identical keys: uniform weights, the output is the mean of the values
    K = np.repeat(rng.standard_normal((nkv, 1, d)).astype(np.float32), L, axis=1)
    o = _f(oracle.attention(q, _bits(K), _bits(V), L))
    mean = _f(_bits(V)).mean(axis=1)
    for h in range(nq):
        np.testing.assert_allclose(o[h], mean[h // 2], rtol=1e-2, atol=1e-2)
    # one key aligned with a large query dominates: the output is its value
    qa = np.zeros((nq, d), np.float32)
    qa[:, 0] = 40.0
    Ka = np.zeros((nkv, L, d), np.float32)
    Ka[:, 5, 0] = 40.0
    o = _f(oracle.attention(_bits(qa), _bits(Ka), _bits(V), L))
    for h in range(nq):
        np.testing.assert_allclose(o[h], _f(_bits(V))[h // 2, 5], atol=1e-2)
    # a single key: the output is that value, exactly
    o = oracle.attention(q, _bits(K), _bits(V), 1)
    for h in range(nq):
        assert np.array_equal(o[h], _bits(V)[h // 2, 0])
    # grouped heads: query heads 2 and 3 read key/value head 1 only
    Vg = np.zeros((nkv, L, d), np.float32)
    Vg[1] = 3.0
    o = _f(oracle.attention(q, _bits(K), _bits(Vg), L))
    assert np.all(o[:2] == 0.0) and np.all(o[2:] == 3.0)
    # entries past L are not read
    V2 = V.copy()
    V2[:, L - 1] = 1e4
    o1 = oracle.attention(q, _bits(K), _bits(V), L - 1)
    o2 = oracle.attention(q, _bits(K), _bits(V2), L - 1)
    assert np.array_equal(o1, o2)


def test_attention_is_invariant_to_the_order_of_the_entries():
    rng = np.random.default_rng(6)
    nq, nkv, d, L = 8, 1, 32, 40
    q = _bits(rng.standard_normal((nq, d)))
    K = _bits(rng.standard_normal((nkv, L, d)))
    V = _bits(rng.standard_normal((nkv, L, d)))
    perm = rng.permutation(L)
    o1 = _f(oracle.attention(q, K, V, L))
    o2 = _f(oracle.attention(q, K[:, perm], V[:, perm], L))
    np.testing.assert_allclose(o1, o2, atol=1e-2)


def _tiny_decoder(seed=0, zero_wo=False, zero_q=False):
    rng = np.random.default_rng(seed)
    T, H, nq, nkv, d, pos, Lcap = 3, 128, 4, 2, 32, 10, 16
    E, k, I = 8, 2, 128
    s = lambda *shape: rng.standard_normal(shape).astype(np.float32)
    g1, g2 = _bits(1 + 0.1 * s(H)), _bits(1 + 0.1 * s(H))
    Wqkv = s((nq + 2 * nkv) * d, H) * 0.1
    if zero_q:
        Wqkv[:nq * d] = 0.0
    Wo = np.zeros((H, nq * d), np.float32) if zero_wo else s(H, nq * d) * 0.1
    kc = np.zeros((T, nkv, Lcap, d), np.float32)
    vc = np.zeros((T, nkv, Lcap, d), np.float32)
    kc[:, :, :pos] = s(T, nkv, pos, d)
    vc[:, :, :pos] = s(T, nkv, pos, d)
    moe = dict(Wr=_bits(s(E, H) * 0.1), W13=_bits(s(E, 2 * I, H) * 0.1), Wd=_bits(s(E, H, I) * 0.1))
    args = dict(x=_bits(s(T, H)), g1=g1, Wqkv=_bits(Wqkv), kcache=_bits(kc), vcache=_bits(vc), Wo=_bits(Wo), g2=g2,
                k=k, nq=nq, nkv=nkv, d=d, pos=pos, **moe)
    return args


def test_decoder_without_attention_output_is_the_moe_block():
    # Wo = 0: the attention block adds nothing, so x2 = x and the layer is
    # x + MoE(RMSNorm(x)), computed here from the (pinned) MoE oracle
    a = _tiny_decoder(zero_wo=True)
    r = oracle.decoder(**a)
    assert np.array_equal(r["x2"], a["x"])
    h2 = oracle.rmsnorm(a["x"], a["g2"])
    m = oracle.moe(h2, a["Wr"], a["W13"], a["Wd"], k=a["k"])
    assert np.array_equal(r["moe_out"], m["out"])
    for key in ("topk_ids", "counts", "exp_indptr", "perm", "slot"):
        assert np.array_equal(r[key], m[key])
    want = wl.to_bf16_bits((_f(a["x"]) + _f(m["out"])).astype(np.float32))
    assert np.array_equal(r["out"], want)


def test_decoder_cache_update_and_uniform_attention():
    # Wq = 0: every score is 0, so each head averages the values of entries
    # 0..pos, the last of which is the new token's own value
    a = _tiny_decoder(zero_q=True)
    r = oracle.decoder(**a)
    T, nq, nkv, d, pos = 3, a["nq"], a["nkv"], a["d"], a["pos"]
    qkv = _f(r["qkv"])
    assert np.all(qkv[:, :nq * d] == 0.0)
    for t in range(T):
        for g in range(nkv):
            # the new key (after RoPE) and value were written at index pos
            assert np.array_equal(r["kcache"][t, g, pos], r["qkv"][t, (nq + g) * d:(nq + g + 1) * d])
            assert np.array_equal(r["vcache"][t, g, pos], r["qkv"][t, (nq + nkv + g) * d:(nq + nkv + g + 1) * d])
            # and no other entry changed
            assert np.array_equal(np.delete(r["kcache"][t, g], pos, 0), np.delete(a["kcache"][t, g], pos, 0))
        att = _f(r["att"])[t].reshape(nq, d)
        for h in range(nq):
            mean = _f(r["vcache"][t, h // (nq // nkv), :pos + 1]).mean(axis=0)
            np.testing.assert_allclose(att[h], mean, rtol=1e-2, atol=1e-2)
    # the projection and residual: a = att Wo^T, x2 = x + a
    np.testing.assert_array_equal(r["a"], oracle.linear(r["att"], a["Wo"]))
    np.testing.assert_array_equal(
        r["x2"], wl.to_bf16_bits((_f(a["x"]) + _f(r["a"])).astype(np.float32)))
