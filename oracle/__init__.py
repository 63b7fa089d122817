"""CPU oracle for the MoE layer and the split-K example.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP path (``dynamic_moe_task_amd``) and never imports it.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64 except the
fixed-order fp32 router contract); this module only compiles it with gcc,
loads it with ctypes and marshals numpy arrays.  ``events.py`` holds a
pure-Python model of the event-tensor runtime for small task graphs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE arithmetic, no fast-math, no FMA
    contraction of separate multiplies and adds)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fopenmp",
            "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_router_logits.argtypes = [i, i, i, P, P, P, P]
        lib.oracle_router_logits_f64.argtypes = [i, i, i, P, P, P, P]
        lib.oracle_topk.argtypes = [i, i, i, P, i, P, P]
        lib.oracle_route_scan.argtypes = [i, i, i, P, P, P, P, P]
        lib.oracle_moe.argtypes = [i, i, i, i, i, i] + [P] * 16
        lib.oracle_moe_tokens.argtypes = [i, i, i, i, P, P, P, P, P, P, P]
        lib.oracle_splitk.argtypes = [i, i, i, P, P, P, P]
        lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        d = ctypes.c_double
        lib.oracle_rmsnorm.argtypes = [i, i, P, P, d, P]
        lib.oracle_linear.argtypes = [i, i, i, P, P, P]
        lib.oracle_rope.argtypes = [i, i, P, d, d]
        lib.oracle_attention.argtypes = [i, i, i, i, i, P, P, P, P]
        lib.oracle_decoder.argtypes = [i, i, i, i, i, i, i, d, d, P, P, P, P, P, P, P, i, i, i, i] + [P] * 18
        lib.oracle_set_threads.argtypes = [i]
        lib.oracle_max_threads.restype = i
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 arrays are passed as their uint16 bit patterns")
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def f32_to_bf16_bits(x: float) -> int:
    return int(_load().oracle_f32_to_bf16(ctypes.c_float(x)))


def bf16_bits_to_f32(b: int) -> float:
    return float(_load().oracle_bf16_to_f32(ctypes.c_uint16(b)))


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (shift into the top half)."""
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def router_logits(X, Wr, bias=None) -> np.ndarray:
    X, Wr = _u16(X), _u16(Wr)
    T, H = X.shape
    E = Wr.shape[0]
    L = np.empty((T, E), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    _check(_load().oracle_router_logits(T, H, E, _p(X), _p(Wr), _p(b), _p(L)), "logits")
    return L


def router_logits_f64(X, Wr, bias=None) -> np.ndarray:
    X, Wr = _u16(X), _u16(Wr)
    T, H = X.shape
    E = Wr.shape[0]
    L = np.empty((T, E), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    _check(_load().oracle_router_logits_f64(T, H, E, _p(X), _p(Wr), _p(b), _p(L)), "logits_f64")
    return L


def topk(L, k: int, norm_topk: bool = True):
    L = np.ascontiguousarray(L, np.float32)
    T, E = L.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(_load().oracle_topk(T, E, k, _p(L), int(norm_topk), _p(ids), _p(w)), "topk")
    return ids, w


def route_scan(ids, E: int):
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    indptr = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    slot = np.empty(T * k, np.int32)
    _check(_load().oracle_route_scan(T, E, k, _p(ids), _p(counts), _p(indptr), _p(perm), _p(slot)),
           "route_scan")
    return counts, indptr, perm, slot


def moe(X, Wr, W13, Wd, k: int, norm_topk: bool = True, bias=None, intermediates: bool = False):
    """Whole layer.  Returns a dict of numpy arrays (bf16 as uint16 bits)."""
    X, Wr, W13, Wd = _u16(X), _u16(Wr), _u16(W13), _u16(Wd)
    T, H = X.shape
    E = Wr.shape[0]
    I = Wd.shape[2]
    assert W13.shape == (E, 2 * I, H) and Wd.shape == (E, H, I)
    r = {
        "logits": np.empty((T, E), np.float32),
        "topk_ids": np.empty((T, k), np.int32),
        "topk_w": np.empty((T, k), np.float32),
        "counts": np.empty(E, np.int32),
        "exp_indptr": np.empty(E + 1, np.int32),
        "perm": np.empty(T * k, np.int32),
        "slot": np.empty(T * k, np.int32),
        "out": np.empty((T, H), np.uint16),
    }
    if intermediates:
        r["Xp"] = np.empty((T * k, H), np.uint16)
        r["Hmid"] = np.empty((T * k, I), np.uint16)
        r["Y"] = np.empty((T * k, H), np.uint16)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    _check(_load().oracle_moe(
        T, H, E, k, I, int(norm_topk), _p(X), _p(Wr), _p(b), _p(W13), _p(Wd),
        _p(r["logits"]), _p(r["topk_ids"]), _p(r["topk_w"]), _p(r["counts"]),
        _p(r["exp_indptr"]), _p(r["perm"]), _p(r["slot"]), _p(r.get("Xp")),
        _p(r.get("Hmid")), _p(r.get("Y")), _p(r["out"])), "moe")
    return r


def route(X, Wr, k: int, norm_topk: bool = True, bias=None):
    """Routing only (logits, top-k, counts, exp_indptr, perm, slot)."""
    L = router_logits(X, Wr, bias)
    ids, w = topk(L, k, norm_topk)
    counts, indptr, perm, slot = route_scan(ids, Wr.shape[0])
    return {"logits": L, "topk_ids": ids, "topk_w": w, "counts": counts,
            "exp_indptr": indptr, "perm": perm, "slot": slot}


def moe_tokens(tokens, X, W13, Wd, topk_ids, topk_w):
    """Output rows of the given tokens from precomputed routing."""
    X, W13, Wd = _u16(X), _u16(W13), _u16(Wd)
    tok = np.ascontiguousarray(tokens, np.int32)
    H = X.shape[1]
    I = Wd.shape[2]
    k = topk_ids.shape[1]
    ids = np.ascontiguousarray(topk_ids, np.int32)
    w = np.ascontiguousarray(topk_w, np.float32)
    out = np.empty((len(tok), H), np.uint16)
    _check(_load().oracle_moe_tokens(H, k, I, len(tok), _p(tok), _p(X), _p(W13), _p(Wd),
                                     _p(ids), _p(w), _p(out)), "moe_tokens")
    return out


# ------------------------------------------------------------ decoder layer --
def rmsnorm(x, g, eps=1e-6):
    x, g = _u16(x), _u16(g)
    T, H = x.shape
    y = np.empty_like(x)
    _check(_load().oracle_rmsnorm(T, H, _p(x), _p(g), float(eps), _p(y)), "rmsnorm")
    return y


def linear(x, W):
    """y = bf16(x W^T), W row-major [N, K]."""
    x, W = _u16(x), _u16(W)
    T, K = x.shape
    N = W.shape[0]
    assert W.shape[1] == K
    y = np.empty((T, N), np.uint16)
    _check(_load().oracle_linear(T, K, N, _p(x), _p(W), _p(y)), "linear")
    return y


def rope(v, pos, theta=1e6):
    """Rotary embedding of the rows of v [n, d] at position pos (returns a copy)."""
    v = np.array(_u16(v), copy=True)
    n, d = v.shape
    _check(_load().oracle_rope(n, d, _p(v), float(pos), float(theta)), "rope")
    return v


def attention(q, Kc, Vc, L):
    """Decode attention of one token: q [nq, d], caches [nkv, Lcap, d]; keys 0..L-1."""
    q, Kc, Vc = _u16(q), _u16(Kc), _u16(Vc)
    nq, d = q.shape
    nkv, Lcap, _ = Kc.shape
    o = np.empty((nq, d), np.uint16)
    _check(_load().oracle_attention(nq, nkv, d, int(L), Lcap, _p(q), _p(Kc), _p(Vc), _p(o)), "attention")
    return o


def decoder(x, g1, Wqkv, kcache, vcache, Wo, g2, Wr, W13, Wd, k, nq, nkv, d, pos, theta=1e6, eps=1e-6,
            norm_topk=True):
    """One decoder layer (attention block, then the MoE block) for the T rows
    of x, each decoding at position pos with its own cache.  The caches are
    copied, updated at index pos and returned with the results."""
    x, g1, Wqkv, Wo, g2 = _u16(x), _u16(g1), _u16(Wqkv), _u16(Wo), _u16(g2)
    Wr, W13, Wd = _u16(Wr), _u16(W13), _u16(Wd)
    kc = np.array(_u16(kcache), copy=True)
    vc = np.array(_u16(vcache), copy=True)
    T, H = x.shape
    E = Wr.shape[0]
    I = Wd.shape[2]
    Lcap = kc.shape[2]
    assert kc.shape == (T, nkv, Lcap, d) and vc.shape == kc.shape
    nqkv = (nq + 2 * nkv) * d
    r = {"logits": np.empty((T, E), np.float32), "topk_ids": np.empty((T, k), np.int32),
         "topk_w": np.empty((T, k), np.float32), "counts": np.empty(E, np.int32),
         "exp_indptr": np.empty(E + 1, np.int32), "perm": np.empty(T * k, np.int32),
         "slot": np.empty(T * k, np.int32), "out": np.empty((T, H), np.uint16),
         "h1": np.empty((T, H), np.uint16), "qkv": np.empty((T, nqkv), np.uint16),
         "att": np.empty((T, nq * d), np.uint16), "a": np.empty((T, H), np.uint16),
         "x2": np.empty((T, H), np.uint16), "h2": np.empty((T, H), np.uint16),
         "moe_out": np.empty((T, H), np.uint16)}
    _check(_load().oracle_decoder(
        T, H, nq, nkv, d, int(pos), Lcap, float(theta), float(eps), _p(x), _p(g1), _p(Wqkv), _p(kc), _p(vc),
        _p(Wo), _p(g2), E, k, I, int(norm_topk), _p(Wr), _p(W13), _p(Wd), _p(r["logits"]), _p(r["topk_ids"]),
        _p(r["topk_w"]), _p(r["counts"]), _p(r["exp_indptr"]), _p(r["perm"]), _p(r["slot"]), _p(r["out"]),
        _p(r["h1"]), _p(r["qkv"]), _p(r["att"]), _p(r["a"]), _p(r["x2"]), _p(r["h2"]), _p(r["moe_out"])),
        "decoder")
    r["kcache"], r["vcache"] = kc, vc
    return r


def set_threads(n: int) -> int:
    """Threads for the per-row loops (OpenMP); returns the count now in force.
    The results do not depend on it."""
    lib = _load()
    lib.oracle_set_threads(int(n))
    return int(lib.oracle_max_threads())


def splitk(A, nsplit: int):
    A = np.ascontiguousarray(A, np.int32)
    n, cols = A.shape
    assert cols % nsplit == 0
    bk = cols // nsplit
    B = np.empty((n, nsplit), np.int32)
    C = np.empty(n, np.int32)
    notif = np.empty(n, np.int32)
    _check(_load().oracle_splitk(n, nsplit, bk, _p(A), _p(B), _p(C), _p(notif)), "splitk")
    return B, C, notif


def expected_tiles(exp_indptr, bm: int):
    """Tile ranges an expert triggers (ET podcast, cue 9): expert e's rows
    [exp_indptr[e], exp_indptr[e+1]) cut into ceil(count/bm) row tiles.
    Returns a list of (e, row_begin, row_end) in expert order."""
    tiles = []
    for e in range(len(exp_indptr) - 1):
        lo, hi = int(exp_indptr[e]), int(exp_indptr[e + 1])
        for r0 in range(lo, hi, bm):
            tiles.append((e, r0, min(r0 + bm, hi)))
    return tiles


def row_rel_err(got_bits, ref_bits) -> np.ndarray:
    """Per-row error max_n |got - ref| / max_n |ref| (inf-norm, row-wise)."""
    g = bf16_bits_to_f64(got_bits)
    r = bf16_bits_to_f64(ref_bits)
    num = np.abs(g - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return num / den
