"""Seeded synthetic workloads for the MoE layer (inputs only, no layer math).

Shapes follow a Qwen3-30B-A3B-shaped MoE layer (hidden 2048, 128 experts,
top-8, expert intermediate 768, SwiGLU) plus a tiny variant.  No trained
weights or datasets are used: every tensor is drawn here.

Recipe.  Every tensor (and every expert slice of the expert weights) has its
own counter-seeded stream ``numpy.random.default_rng((seed, tag, ...))``, so
slices can be drawn in parallel and any one of them regenerated alone:
  router weight Wr [E, H]           tag 0          ~ N(0, 0.02)
  W13[e] [2I, H] (gate rows 0..I-1,
          up rows I..2I-1)          tag (1, e)     ~ N(0, 0.02)
  Wd[e] [H, I]                      tag (2, e)     ~ N(0, 0.02)
  activations X [T, H]              tag 3          ~ N(0, 1)
  (Zipf-biased prefill only) rank permutation r = 1 + permutation(E),
                                    tag 4; the per-expert logit offset is
     b_e = -s * ln(r_e) with s = 1.1, i.e. the log of a Zipf(s) pmf up to its
     normaliser, so a few experts draw most tokens and some draw none.
Normals are drawn as float32 and rounded to bf16 (round to nearest, ties to
even); bf16 tensors are held as their uint16 bit patterns.

The batch-size sweep draws B ~ U{1..512} for 200 steps from
``default_rng((seed, 5))`` and the step-s activations from
``default_rng((seed, 6, s))``.

The decoder layer around the MoE layer (batch 8 at decode, 32 query heads,
4 key/value heads of 128, a bf16 KV cache holding 4096 earlier positions per
sequence, then the same 128-expert MoE) draws:
  RMSNorm weights g1, g2 [H]           tags 7, 8      ~ N(1, 0.05)
  Wqkv [(nq + 2 nkv) d, H]             tag 9          ~ N(0, 0.02)
  Wo [H, nq d]                         tag 10         ~ N(0, 0.02)
  key / value caches [T, nkv, Lcap, d] tags 11, 12    ~ N(0, 1)
  residual input x [T, H]              tag 13         ~ N(0, 1)
and the MoE weights of make_weights with the same seed.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class MoEShape:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    norm_topk: bool = True
    zipf_s: Optional[float] = None  # logit offset b_e = -s ln(rank_e)


TINY = MoEShape("tiny T=4 H=128 E=8 k=2 I=256", T=4, H=128, E=8, k=2, I=256)
DECODE = MoEShape("qwen3-30b-a3b moe decode T=16", T=16, H=2048, E=128, k=8, I=768)
PREFILL_ZIPF = MoEShape("qwen3-30b-a3b moe prefill T=256 zipf1.1", T=256, H=2048, E=128, k=8,
                        I=768, zipf_s=1.1)
SWEEP = MoEShape("qwen3-30b-a3b moe sweep B~U[1,512]", T=512, H=2048, E=128, k=8, I=768)
SHAPES = {"tiny": TINY, "decode": DECODE, "prefill_zipf": PREFILL_ZIPF, "sweep": SWEEP}
# Qwen-shape layer at the largest token count of the pages' MoE-layer table
# (the batch where the grouped GEMM nears the matrix-core ridge)
LARGE = MoEShape("qwen3-30b-a3b moe T=4096", T=4096, H=2048, E=128, k=8, I=768)

# Dense MLPs of the pages' appendix table of MLP configurations (sequence
# length S, hidden H, intermediate I of five public models), run through the
# MoE path as one expert that every token picks (E = 1, k = 1: the top-k
# weight renormalises to 1 and the layer is the dense SwiGLU MLP).
MLP_TABLE = [
    MoEShape("MLP-1 (Qwen3-8B) S=8192", T=8192, H=4096, E=1, k=1, I=12288),
    MoEShape("MLP-2 (LLaMA-3.1-8B) S=8192", T=8192, H=4096, E=1, k=1, I=14336),
    MoEShape("MLP-3 (Gemma-2-9B) S=8192", T=8192, H=3584, E=1, k=1, I=14336),
    MoEShape("MLP-4 (Gemma-2-27B) S=8192", T=8192, H=4608, E=1, k=1, I=36864),
    MoEShape("MLP-5 (Qwen3-32B) S=8192", T=8192, H=5120, E=1, k=1, I=25600),
]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(rng, shape, std):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


@dataclass
class MoEWeights:
    Wr: np.ndarray      # [E, H] bf16 bits
    W13: np.ndarray     # [E, 2I, H]
    Wd: np.ndarray      # [E, H, I]
    bias: Optional[np.ndarray] = None  # [E] float32 or None
    seed: int = 0


def make_weights(shape: MoEShape, seed: int = 0, w_std: float = 0.02, threads: int = 8) -> MoEWeights:
    from concurrent.futures import ThreadPoolExecutor
    E, H, I = shape.E, shape.H, shape.I
    Wr = _normal_bf16(np.random.default_rng((seed, 0)), (E, H), w_std)
    W13 = np.empty((E, 2 * I, H), np.uint16)
    Wd = np.empty((E, H, I), np.uint16)

    def fill(e):
        W13[e] = _normal_bf16(np.random.default_rng((seed, 1, e)), (2 * I, H), w_std)
        Wd[e] = _normal_bf16(np.random.default_rng((seed, 2, e)), (H, I), w_std)

    # one expert (the dense MLPs): its rows in blocks, one generator a block,
    # so that the threads share the work
    blk = 1024

    def fill_rows(job):
        which, r0 = job
        if which == 1:
            W13[0, r0:r0 + blk] = _normal_bf16(np.random.default_rng((seed, 1, 0, r0)), W13[0, r0:r0 + blk].shape, w_std)
        else:
            Wd[0, r0:r0 + blk] = _normal_bf16(np.random.default_rng((seed, 2, 0, r0)), Wd[0, r0:r0 + blk].shape, w_std)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        if E == 1:
            jobs = [(1, r) for r in range(0, 2 * I, blk)] + [(2, r) for r in range(0, H, blk)]
            list(ex.map(fill_rows, jobs))
        else:
            list(ex.map(fill, range(E)))
    return MoEWeights(Wr, W13, Wd, None, seed)


def make_tokens(shape: MoEShape, T: int, seed: int = 0) -> np.ndarray:
    return _normal_bf16(np.random.default_rng((seed, 3)), (T, shape.H), 1.0)


def zipf_bias(shape: MoEShape, seed: int = 0) -> Optional[np.ndarray]:
    if shape.zipf_s is None:
        return None
    ranks = 1 + np.random.default_rng((seed, 4)).permutation(shape.E)
    return (-shape.zipf_s * np.log(ranks.astype(np.float64))).astype(np.float32)


def make_layer(shape: MoEShape, seed: int = 0):
    """Weights (with the Zipf bias when the shape has one) and X [T, H]."""
    w = make_weights(shape, seed)
    w.bias = zipf_bias(shape, seed)
    return w, make_tokens(shape, shape.T, seed)


@dataclass(frozen=True)
class DecoderShape:
    name: str
    T: int          # tokens (sequences) decoding together
    H: int
    nq: int         # query heads
    nkv: int        # key / value heads
    d: int          # head size
    pos: int        # position of the new token (= earlier entries in each cache)
    Lcap: int       # cache capacity per sequence and head
    theta: float
    eps: float
    moe: MoEShape


DECODER = DecoderShape("qwen3-30b-a3b decoder layer decode B=8 kv=4096", T=8, H=2048, nq=32, nkv=4, d=128,
                       pos=4096, Lcap=4160, theta=1e6, eps=1e-6,
                       moe=MoEShape("qwen3-30b-a3b moe T=8", T=8, H=2048, E=128, k=8, I=768))


@dataclass
class DecoderWeights:
    g1: np.ndarray    # [H] bf16 bits
    Wqkv: np.ndarray  # [(nq + 2 nkv) d, H]
    Wo: np.ndarray    # [H, nq d]
    g2: np.ndarray    # [H]
    moe: MoEWeights


def make_decoder(shape: DecoderShape, seed: int = 0, w_std: float = 0.02, moe: Optional[MoEWeights] = None):
    """Weights, the residual input x [T, H] and the key / value caches
    [T, nkv, Lcap, d] (entries 0..pos-1 drawn, the rest zero)."""
    H, d = shape.H, shape.d
    nqkv = (shape.nq + 2 * shape.nkv) * d
    g1 = to_bf16_bits(1.0 + 0.05 * np.random.default_rng((seed, 7)).standard_normal(H, dtype=np.float32))
    g2 = to_bf16_bits(1.0 + 0.05 * np.random.default_rng((seed, 8)).standard_normal(H, dtype=np.float32))
    Wqkv = _normal_bf16(np.random.default_rng((seed, 9)), (nqkv, H), w_std)
    Wo = _normal_bf16(np.random.default_rng((seed, 10)), (H, shape.nq * d), w_std)
    cshape = (shape.T, shape.nkv, shape.Lcap, d)
    kc = np.zeros(cshape, np.uint16)
    vc = np.zeros(cshape, np.uint16)
    kc[:, :, :shape.pos] = _normal_bf16(np.random.default_rng((seed, 11)), (shape.T, shape.nkv, shape.pos, d), 1.0)
    vc[:, :, :shape.pos] = _normal_bf16(np.random.default_rng((seed, 12)), (shape.T, shape.nkv, shape.pos, d), 1.0)
    x = _normal_bf16(np.random.default_rng((seed, 13)), (shape.T, H), 1.0)
    if moe is None:
        moe = make_weights(shape.moe, seed)
    return DecoderWeights(g1, Wqkv, Wo, g2, moe), x, kc, vc


def decoder_algorithmic_bytes(shape: DecoderShape, n_active: int) -> int:
    """Bytes the decoder layer must move: the attention weights, the cache
    entries read (pos per sequence and kv head, keys and values) and written
    (the new entry), the norm weights, activations in and out, and the MoE
    block's algorithmic bytes."""
    H, d, T = shape.H, shape.d, shape.T
    w_att = 2 * ((shape.nq + 2 * shape.nkv) * d * H + H * shape.nq * d + 2 * H)
    kv = 2 * 2 * T * shape.nkv * d * (shape.pos + 1)
    return w_att + kv + 2 * T * H * 2 + algorithmic_bytes(shape.moe, T, n_active) - 2 * 2 * T * H


def sweep_batches(seed: int = 0, steps: int = 200, bmax: int = 512) -> np.ndarray:
    return np.random.default_rng((seed, 5)).integers(1, bmax + 1, size=steps)


def sweep_tokens(shape: MoEShape, step: int, B: int, seed: int = 0) -> np.ndarray:
    return _normal_bf16(np.random.default_rng((seed, 6, step)), (B, shape.H), 1.0)


def algorithmic_bytes(shape: MoEShape, T: int, n_active: int) -> int:
    """Bytes the layer must move: router weight, activations in and out,
    and the weights of every expert that received a token."""
    H, E, I = shape.H, shape.E, shape.I
    return 2 * E * H + 2 * T * H + 6 * H * I * n_active + 2 * T * H


def algorithmic_flops(shape: MoEShape, T: int) -> int:
    H, E, I, k = shape.H, shape.E, shape.I, shape.k
    return 2 * T * E * H + 6 * T * k * H * I
