"""Thin ctypes binding of libetc.so (include/etc.h), same names as the C ABI.

Argument marshalling only: every step of the MoE layer runs in the HIP
kernels behind the library.  torch is used for device memory and streams
(pointers come from ``tensor.data_ptr()``, streams from
``torch.cuda.current_stream().cuda_stream``).  If the library is missing this
module raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libetc.so")

ETC_OK = 0
ETC_ERR_INVALID = -1
ETC_ERR_UNSUPPORTED = -2
ETC_ERR_HIP = -3
ETC_ERR_TIMEOUT = -4
ETC_ERR_INVARIANT = -5
ETC_ERR_NONFINITE = -6

ETC_SCHED_STATIC = 0
ETC_SCHED_DYNAMIC = 1
ETC_SCHED_KBK = 2
ETC_SCHED_BARRIER = 3
ETC_SCHED_ORDERED = 4
SCHEDS = {"static": ETC_SCHED_STATIC, "dynamic": ETC_SCHED_DYNAMIC, "kbk": ETC_SCHED_KBK,
          "barrier": ETC_SCHED_BARRIER, "ordered": ETC_SCHED_ORDERED}

ETC_DIM_SYMBOLIC = -1
ETC_WAIT_DATA_DEPENDENT = -1
ETC_MAX_DIMS = 8

EXPORTED = [
    "etensor_create", "etensor_instantiate", "etensor_shape", "etensor_destroy",
    "etc_edge_compile", "etc_edge_index", "etc_splitk_launch", "moe_layer_info", "moe_layer_workspace_size", "moe_workspace_init",
    "moe_layer_launch", "moe_layer_launch_noalloc", "decoder_layer_workspace_size", "decoder_workspace_init",
    "decoder_layer_launch", "etc_coherence_selftest_bytes", "etc_coherence_selftest", "etc_sync", "etc_last_error",
]


class EtcError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"etc error {code}: {msg}")
        self.code = code


class Edge(ctypes.Structure):
    """etc_edge: an edge spec compiled against an event tensor and a task grid."""
    _fields_ = [("task_ndim", ctypes.c_int32), ("event_ndim", ctypes.c_int32),
                ("src", ctypes.c_int32 * ETC_MAX_DIMS), ("stride", ctypes.c_int64 * ETC_MAX_DIMS),
                ("task_shape", ctypes.c_int64 * ETC_MAX_DIMS), ("event_numel", ctypes.c_int64),
                ("fan_in", ctypes.c_int64)]


class MoeDesc(ctypes.Structure):
    _fields_ = [("T_max", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("norm_topk", ctypes.c_int32),
                ("has_bias", ctypes.c_int32)]


class MoeArgs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w_router", ctypes.c_void_p), ("b_router", ctypes.c_void_p),
                ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("exp_indptr", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("slot", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("debug", ctypes.c_void_p), ("watchdog_us", ctypes.c_uint32),
                ("trace_records", ctypes.c_uint32), ("trace", ctypes.c_void_p)]


class DecoderDesc(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("L_cap", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("moe", MoeDesc)]


class DecoderArgs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("g1", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p), ("g2", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("moe", MoeArgs)]


class MoeInfo(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn1", ctypes.c_int32), ("bn2", ctypes.c_int32),
                ("router_tokens", ctypes.c_int32), ("router_experts", ctypes.c_int32),
                ("dispatch_tokens", ctypes.c_int32), ("combine_tokens", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("wall_clock_khz", ctypes.c_int32), ("router_experts_large", ctypes.c_int32),
                ("router_large_from", ctypes.c_int32), ("bn1_large", ctypes.c_int32),
                ("bn1_large_from_rows", ctypes.c_int32), ("bn2_large", ctypes.c_int32),
                ("bn1_mid", ctypes.c_int32), ("bn1_mid_from_rows", ctypes.c_int32),
                ("router_experts_xl", ctypes.c_int32), ("router_xl_from", ctypes.c_int32),
                ("big_from_rows", ctypes.c_int32), ("bm_big", ctypes.c_int32), ("bn1_big", ctypes.c_int32),
                ("bn2_big", ctypes.c_int32), ("grid_big", ctypes.c_int32), ("lds_bytes_big", ctypes.c_int32)]

    def big_for(self, T: int, k: int) -> bool:
        """Whether a launch at batch T, top-k k runs the big-tile variant."""
        return self.big_from_rows > 0 and T * k >= self.big_from_rows

    def bm_for(self, T: int, k: int) -> int:
        """Grouped rows per row tile at batch T, top-k k."""
        return self.bm_big if self.big_for(T, k) else self.bm

    def grid_for(self, T: int, k: int) -> int:
        """Persistent workgroups of a launch at batch T, top-k k."""
        return self.grid_big if self.big_for(T, k) else self.grid

    def router_experts_for(self, T: int) -> int:
        """Experts per router task at batch T."""
        if T >= self.router_xl_from:
            return self.router_experts_xl
        return self.router_experts if T <= self.router_large_from else self.router_experts_large

    def bn1_for(self, T: int, k: int) -> int:
        """Gate (and up) columns per G1 tile at batch T, top-k k."""
        if self.big_for(T, k):
            return self.bn1_big
        if T * k >= self.bn1_large_from_rows:
            return self.bn1_large
        return self.bn1_mid if T * k >= self.bn1_mid_from_rows else self.bn1

    def bn2_for(self, T: int, k: int) -> int:
        """Output columns per G2 tile at batch T, top-k k."""
        if self.big_for(T, k):
            return self.bn2_big
        return self.bn2_large if T * k >= self.bn1_large_from_rows else self.bn2


_lib = None


def lib():
    """Load libetc.so (built by ``python -m dynamic_moe_task_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m dynamic_moe_task_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.etensor_create.argtypes = [ctypes.POINTER(P), ctypes.c_int, ctypes.POINTER(I64), I32, P]
        L.etensor_instantiate.argtypes = [P, ctypes.POINTER(I64)]
        L.etensor_shape.argtypes = [P, ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_int), ctypes.POINTER(I64)]
        L.etensor_destroy.argtypes = [P]
        L.etc_edge_compile.argtypes = [P, ctypes.c_char_p, ctypes.POINTER(I64), ctypes.c_int, ctypes.POINTER(Edge)]
        L.etc_edge_index.argtypes = [ctypes.POINTER(Edge), ctypes.POINTER(I64)]
        L.etc_edge_index.restype = I64
        L.etc_splitk_launch.argtypes = [P, I32, I32, I32, P, P, P, ctypes.POINTER(Edge), ctypes.POINTER(Edge),
                                        ctypes.c_int, P]
        L.moe_layer_info.argtypes = [ctypes.POINTER(MoeDesc), ctypes.POINTER(MoeInfo)]
        L.moe_layer_workspace_size.argtypes = [ctypes.POINTER(MoeDesc)]
        L.moe_layer_workspace_size.restype = ctypes.c_size_t
        L.moe_workspace_init.argtypes = [ctypes.POINTER(MoeDesc), P, ctypes.c_size_t, P]
        L.moe_layer_launch.argtypes = [ctypes.POINTER(MoeDesc), I32, ctypes.POINTER(MoeArgs), ctypes.c_int, P]
        L.moe_layer_launch_noalloc.argtypes = [ctypes.POINTER(MoeDesc), I32, ctypes.POINTER(MoeArgs), ctypes.c_int, P]
        L.decoder_layer_workspace_size.argtypes = [ctypes.POINTER(DecoderDesc)]
        L.decoder_layer_workspace_size.restype = ctypes.c_size_t
        L.decoder_workspace_init.argtypes = [ctypes.POINTER(DecoderDesc), P, ctypes.c_size_t, P]
        L.decoder_layer_launch.argtypes = [ctypes.POINTER(DecoderDesc), I32, I32, ctypes.POINTER(DecoderArgs),
                                           ctypes.c_int, P]
        L.etc_sync.argtypes = [P]
        L.etc_coherence_selftest_bytes.argtypes = [I32]
        L.etc_coherence_selftest_bytes.restype = ctypes.c_size_t
        L.etc_coherence_selftest.argtypes = [I32, I32, P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_uint32), P]
        L.etc_last_error.argtypes = []
        L.etc_last_error.restype = ctypes.c_char_p
        for name in ["etensor_create", "etensor_instantiate", "etensor_shape", "etensor_destroy",
                     "etc_edge_compile", "etc_splitk_launch", "moe_layer_info", "moe_workspace_init", "moe_layer_launch",
                     "moe_layer_launch_noalloc", "decoder_workspace_init", "decoder_layer_launch",
                     "etc_sync"]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def etc_last_error() -> str:
    return lib().etc_last_error().decode()


def check(rc: int) -> int:
    if rc != ETC_OK:
        raise EtcError(rc, etc_last_error())
    return rc


# ------------------------------------------------------------ event tensors --
def etensor_create(shape, wait_count: int, dev_counters: Optional[int] = None):
    h = ctypes.c_void_p()
    arr = (ctypes.c_int64 * len(shape))(*shape)
    check(lib().etensor_create(ctypes.byref(h), len(shape), arr, wait_count, dev_counters))
    return h


def etensor_instantiate(h, concrete_shape) -> None:
    arr = (ctypes.c_int64 * len(concrete_shape))(*concrete_shape)
    check(lib().etensor_instantiate(h, arr))


def etensor_shape(h):
    shp = (ctypes.c_int64 * ETC_MAX_DIMS)()
    nd = ctypes.c_int()
    numel = ctypes.c_int64()
    check(lib().etensor_shape(h, shp, ctypes.byref(nd), ctypes.byref(numel)))
    return tuple(shp[i] for i in range(nd.value)), numel.value


def etensor_destroy(h) -> None:
    check(lib().etensor_destroy(h))


def etc_edge_compile(ev, spec: str, task_shape) -> Edge:
    e = Edge()
    arr = (ctypes.c_int64 * len(task_shape))(*task_shape)
    check(lib().etc_edge_compile(ev, spec.encode(), arr, len(task_shape), ctypes.byref(e)))
    return e


def etc_edge_index(edge: Edge, coord) -> int:
    arr = (ctypes.c_int64 * len(coord))(*coord)
    return int(lib().etc_edge_index(ctypes.byref(edge), arr))


def etc_splitk_launch(ev, n, nsplit, bk, A_ptr, B_ptr, C_ptr, notify_edge: Edge, wait_edge: Edge, sched,
                      stream) -> int:
    return lib().etc_splitk_launch(ev, n, nsplit, bk, A_ptr, B_ptr, C_ptr, ctypes.byref(notify_edge),
                                   ctypes.byref(wait_edge), sched, stream)


# ---------------------------------------------------------------- MoE layer --
def moe_desc(T_max, H, E, k, I, norm_topk=True, has_bias=False) -> MoeDesc:
    return MoeDesc(T_max, H, E, k, I, int(bool(norm_topk)), int(bool(has_bias)))


def moe_layer_workspace_size(desc: MoeDesc) -> int:
    return lib().moe_layer_workspace_size(ctypes.byref(desc))


def trace_words(records: int) -> int:
    """ETC_TRACE_WORDS: uint32 words of a trace buffer holding `records`."""
    return 16 + 8 * int(records)


def moe_layer_info(desc: MoeDesc) -> MoeInfo:
    info = MoeInfo()
    check(lib().moe_layer_info(ctypes.byref(desc), ctypes.byref(info)))
    return info


def moe_workspace_init(desc: MoeDesc, ws_ptr: int, ws_bytes: int, stream) -> int:
    return lib().moe_workspace_init(ctypes.byref(desc), ws_ptr, ws_bytes, stream)


def moe_layer_launch(desc: MoeDesc, T: int, args: MoeArgs, sched: int, stream) -> int:
    return lib().moe_layer_launch(ctypes.byref(desc), T, ctypes.byref(args), sched, stream)


def moe_layer_launch_noalloc(desc: MoeDesc, T: int, args: MoeArgs, sched: int, stream) -> int:
    return lib().moe_layer_launch_noalloc(ctypes.byref(desc), T, ctypes.byref(args), sched, stream)


def decoder_desc(T_max, H, n_q, n_kv, head_dim, L_cap, E, k, I, rope_theta=1e6, rms_eps=1e-6,
                 norm_topk=True) -> DecoderDesc:
    return DecoderDesc(n_q, n_kv, head_dim, L_cap, rope_theta, rms_eps, moe_desc(T_max, H, E, k, I, norm_topk, False))


def decoder_layer_workspace_size(desc: DecoderDesc) -> int:
    return lib().decoder_layer_workspace_size(ctypes.byref(desc))


def decoder_workspace_init(desc: DecoderDesc, ws_ptr: int, ws_bytes: int, stream) -> int:
    return lib().decoder_workspace_init(ctypes.byref(desc), ws_ptr, ws_bytes, stream)


def decoder_layer_launch(desc: DecoderDesc, T: int, pos: int, args: DecoderArgs, sched: int, stream) -> int:
    return lib().decoder_layer_launch(ctypes.byref(desc), T, pos, ctypes.byref(args), sched, stream)


def etc_sync(stream) -> int:
    return lib().etc_sync(stream)


def etc_coherence_selftest_bytes(pairs: int) -> int:
    return int(lib().etc_coherence_selftest_bytes(pairs))


def etc_coherence_selftest(pairs: int, rounds: int, workspace_ptr: int, workspace_bytes: int, stream) -> tuple:
    """Runs the cross-workgroup message-passing self-test; returns
    (words read wrong, wait gave up) from the library's result words."""
    res = (ctypes.c_uint32 * 2)()
    check(lib().etc_coherence_selftest(pairs, rounds, workspace_ptr, workspace_bytes, res, stream))
    return int(res[0]), int(res[1])


@dataclass
class MoELayerBuffers:
    """Device tensors of one MoE layer, owned by torch, handed to the library
    as raw pointers.  bf16 tensors are torch.bfloat16."""
    desc: MoeDesc
    x: object
    w_router: object
    b_router: object
    w13: object
    w2: object
    out: object
    topk_ids: object
    topk_w: object
    counts: object
    exp_indptr: object
    perm: object
    slot: object
    workspace: object
    debug: object = None

    @staticmethod
    def allocate(desc: MoeDesc, w_router, w13, w2, b_router=None, device="cuda", debug=False):
        import torch
        Tm, H, E, k = desc.T_max, desc.H, desc.E, desc.k
        i32 = dict(dtype=torch.int32, device=device)
        ws_bytes = moe_layer_workspace_size(desc)
        if ws_bytes == 0:
            raise EtcError(ETC_ERR_INVALID, etc_last_error())
        bufs = MoELayerBuffers(
            desc=desc,
            x=torch.empty((Tm, H), dtype=torch.bfloat16, device=device),
            w_router=w_router, b_router=b_router, w13=w13, w2=w2,
            out=torch.empty((Tm, H), dtype=torch.bfloat16, device=device),
            topk_ids=torch.empty((Tm, k), **i32),
            topk_w=torch.empty((Tm, k), dtype=torch.float32, device=device),
            counts=torch.empty(E, **i32),
            exp_indptr=torch.empty(E + 1, **i32),
            perm=torch.empty(Tm * k, **i32),
            slot=torch.empty(Tm * k, **i32),
            workspace=torch.zeros(ws_bytes, dtype=torch.uint8, device=device),
            debug=torch.zeros(2 * E + 8, **i32) if debug else None,
        )
        stream = torch.cuda.current_stream().cuda_stream
        check(moe_workspace_init(desc, bufs.workspace.data_ptr(), ws_bytes, stream))
        return bufs

    def args(self, x=None, w13=None, w2=None, watchdog_us: int = 0, trace=None) -> MoeArgs:
        x = self.x if x is None else x
        w13 = self.w13 if w13 is None else w13
        w2 = self.w2 if w2 is None else w2
        return MoeArgs(
            x.data_ptr(), self.w_router.data_ptr(),
            self.b_router.data_ptr() if self.b_router is not None else None,
            w13.data_ptr(), w2.data_ptr(), self.out.data_ptr(), self.topk_ids.data_ptr(),
            self.topk_w.data_ptr(), self.counts.data_ptr(), self.exp_indptr.data_ptr(),
            self.perm.data_ptr(), self.slot.data_ptr(), self.workspace.data_ptr(),
            self.workspace.numel(), self.debug.data_ptr() if self.debug is not None else None,
            watchdog_us, 0 if trace is None else (trace.numel() - 16) // 8,
            None if trace is None else trace.data_ptr())

    def launch(self, T: int, sched="static", stream=None, **kw) -> None:
        import torch
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        check(moe_layer_launch(self.desc, T, self.args(**kw), SCHEDS.get(sched, sched), s))


@dataclass
class DecoderBuffers:
    """Device tensors of one decoder layer (weights, caches, the MoE block's
    buffers and the workspace), owned by torch, handed over as pointers."""
    desc: DecoderDesc
    x: object
    g1: object
    w_qkv: object
    w_o: object
    g2: object
    k_cache: object
    v_cache: object
    moe: MoELayerBuffers

    @staticmethod
    def allocate(desc: DecoderDesc, g1, w_qkv, w_o, g2, k_cache, v_cache, w_router, w13, w2, device="cuda",
                 debug=False):
        import torch
        Tm, H, E, k = desc.moe.T_max, desc.moe.H, desc.moe.E, desc.moe.k
        i32 = dict(dtype=torch.int32, device=device)
        ws_bytes = decoder_layer_workspace_size(desc)
        if ws_bytes == 0:
            raise EtcError(ETC_ERR_INVALID, etc_last_error())
        moe = MoELayerBuffers(
            desc=desc.moe, x=torch.empty((Tm, H), dtype=torch.bfloat16, device=device),
            w_router=w_router, b_router=None, w13=w13, w2=w2,
            out=torch.empty((Tm, H), dtype=torch.bfloat16, device=device),
            topk_ids=torch.empty((Tm, k), **i32), topk_w=torch.empty((Tm, k), dtype=torch.float32, device=device),
            counts=torch.empty(E, **i32), exp_indptr=torch.empty(E + 1, **i32), perm=torch.empty(Tm * k, **i32),
            slot=torch.empty(Tm * k, **i32), workspace=torch.zeros(ws_bytes, dtype=torch.uint8, device=device),
            debug=torch.zeros(2 * E + 8, **i32) if debug else None)
        stream = torch.cuda.current_stream().cuda_stream
        check(decoder_workspace_init(desc, moe.workspace.data_ptr(), ws_bytes, stream))
        x = torch.empty((Tm, H), dtype=torch.bfloat16, device=device)
        return DecoderBuffers(desc, x, g1, w_qkv, w_o, g2, k_cache, v_cache, moe)

    def args(self, w13=None, w2=None, w_qkv=None, w_o=None, k_cache=None, v_cache=None, watchdog_us: int = 0,
             trace=None) -> DecoderArgs:
        pick = lambda a, b: b if a is None else a
        return DecoderArgs(self.x.data_ptr(), self.g1.data_ptr(), pick(w_qkv, self.w_qkv).data_ptr(),
                           pick(w_o, self.w_o).data_ptr(), self.g2.data_ptr(),
                           pick(k_cache, self.k_cache).data_ptr(), pick(v_cache, self.v_cache).data_ptr(),
                           self.moe.args(w13=w13, w2=w2, watchdog_us=watchdog_us, trace=trace))

    def launch(self, T: int, pos: int, sched="static", stream=None, **kw) -> None:
        import torch
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        check(decoder_layer_launch(self.desc, T, pos, self.args(**kw), SCHEDS.get(sched, sched), s))
