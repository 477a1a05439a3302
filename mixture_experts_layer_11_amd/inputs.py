"""Seeded synthetic inputs for the MoE layer forward.

This module only *makes inputs*: it draws the tokens, the router weight, the
selection bias and the SwiGLU expert weights, and stores them in the formats
the layer consumes (fp32 values, bf16 bit patterns, or OCP e4m3fn codes with
one fp32 scale per 128x128 weight block).  It holds no step of the layer's own
arithmetic; the oracle and the HIP path both read what it produces and share
nothing else.

Layer shapes follow the DeepSeek-V3.2-Exp pages: x [B,T,7168] flattened to
[T,dim] ("Weighted expert sum", in/out shapes), router weight [E,dim] held as
[out,in] ("Expert scores", parameter accounting), 256 routed experts, top-8.
Expert internals (SwiGLU with w1/w3 [inter,dim], w2 [dim,inter]), the fp8
block scheme and the value distributions are the plainest reading of the
workload descriptions and are listed with each config below.

Random streams: numpy ``Generator(PCG64)`` seeded with
``[seed, tensor_tag, expert_id]``, so every tensor and every expert is an
independent stream and experts can be drawn in any order or in parallel.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

# tensor tags of the random streams
TAG_X, TAG_WR, TAG_BIAS, TAG_W1, TAG_W3, TAG_W2, TAG_WS1, TAG_WS3, TAG_WS2, TAG_HOT = range(10)

FP8_BLOCK = 128  # weight scales cover 128x128 blocks, activation scales 1x128


@dataclass(frozen=True)
class MoEConfig:
    """One synthetic workload.

    act_dtype: dtype of x and of y ("f32" or "bf16").
    w_dtype:   dtype of routed and shared expert weights ("f32", "bf16", "fp8").
    router_dtype: dtype of the router weight ("f32" or "bf16"); applied in fp32.
    bias_range: selection bias ~U(-r, r) in fp32, or None for no bias.
    inter_shared: inner width of the one shared SwiGLU MLP (0 = no shared expert).
    hot_experts/hot_scale: that many router rows (chosen by a seeded draw) are
        multiplied by hot_scale after rounding, to skew the load.
    """

    name: str
    T: int
    dim: int
    E: int
    n_groups: int
    topk_groups: int
    topk: int
    score_func: str
    route_scale: float
    bias_range: Optional[float]
    inter: int
    inter_shared: int
    act_dtype: str
    w_dtype: str
    router_dtype: str
    seed: int
    hot_experts: int = 0
    hot_scale: float = 1.0

    def with_T(self, T: int) -> "MoEConfig":
        return replace(self, T=T, name=f"{self.name}@T{T}")


# The five workloads.  c1/c2/c4 are the DeepSeek-V3 layer shape (dim 7168,
# 256 experts in 8 groups, 4 groups kept, top-8, route_scale 2.5, expert inner
# width 2048, one shared expert of the same width).
CONFIGS = [
    MoEConfig("c0_tiny_fp32", T=64, dim=256, E=16, n_groups=4, topk_groups=2, topk=4,
              score_func="sigmoid", route_scale=1.0, bias_range=0.1, inter=128,
              inter_shared=128, act_dtype="f32", w_dtype="f32", router_dtype="f32",
              seed=11000),
    MoEConfig("c1_dsv3_decode_T128", T=128, dim=7168, E=256, n_groups=8, topk_groups=4,
              topk=8, score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=2048,
              inter_shared=2048, act_dtype="bf16", w_dtype="bf16", router_dtype="bf16",
              seed=11001),
    MoEConfig("c2_dsv3_prefill_T4096", T=4096, dim=7168, E=256, n_groups=8, topk_groups=4,
              topk=8, score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=2048,
              inter_shared=2048, act_dtype="bf16", w_dtype="bf16", router_dtype="bf16",
              seed=11002),
    MoEConfig("c3_skewed_softmax_T8192", T=8192, dim=2048, E=64, n_groups=1, topk_groups=1,
              topk=6, score_func="softmax", route_scale=1.0, bias_range=None, inter=1408,
              inter_shared=2 * 1408, act_dtype="bf16", w_dtype="bf16", router_dtype="bf16",
              seed=11003, hot_experts=8, hot_scale=4.0),
    MoEConfig("c4_dsv3_fp8_T8192", T=8192, dim=7168, E=256, n_groups=8, topk_groups=4,
              topk=8, score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=2048,
              inter_shared=2048, act_dtype="bf16", w_dtype="fp8", router_dtype="bf16",
              seed=11004),
]

# Small shapes for parity tests: several MFMA tiles, ragged token counts.
SMALL_CONFIGS = [
    next(c for c in CONFIGS if c.name == "c0_tiny_fp32"),
    MoEConfig("s1_mini_dsv3_bf16", T=333, dim=512, E=32, n_groups=4, topk_groups=2, topk=4,
              score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=256,
              inter_shared=256, act_dtype="bf16", w_dtype="bf16", router_dtype="bf16",
              seed=12001),
    MoEConfig("s2_mini_softmax_hot", T=517, dim=256, E=16, n_groups=1, topk_groups=1, topk=3,
              score_func="softmax", route_scale=1.0, bias_range=None, inter=192,
              inter_shared=384, act_dtype="bf16", w_dtype="bf16", router_dtype="bf16",
              seed=12002, hot_experts=2, hot_scale=4.0),
    MoEConfig("s3_mini_fp8", T=300, dim=256, E=16, n_groups=4, topk_groups=2, topk=4,
              score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=256,
              inter_shared=256, act_dtype="bf16", w_dtype="fp8", router_dtype="bf16",
              seed=12003),
    MoEConfig("s4_mini_decode_bf16", T=24, dim=1024, E=64, n_groups=8, topk_groups=4, topk=8,
              score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=512,
              inter_shared=512, act_dtype="bf16", w_dtype="bf16", router_dtype="bf16",
              seed=12004),
    MoEConfig("s5_mini_prefill_bf16", T=1000, dim=640, E=16, n_groups=4, topk_groups=2, topk=4,
              score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=384,
              inter_shared=256, act_dtype="bf16", w_dtype="bf16", router_dtype="bf16",
              seed=12005),
    MoEConfig("s6_mini_prefill_odd", T=700, dim=448, E=16, n_groups=4, topk_groups=2, topk=4,
              score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=320,
              inter_shared=192, act_dtype="bf16", w_dtype="bf16", router_dtype="bf16",
              seed=12006),
    MoEConfig("s7_mini_fp8_decode", T=40, dim=768, E=32, n_groups=4, topk_groups=2, topk=4,
              score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=384,
              inter_shared=256, act_dtype="bf16", w_dtype="fp8", router_dtype="bf16",
              seed=12007),
    MoEConfig("s8_mini_fp8_prefill_ragged", T=900, dim=384, E=8, n_groups=2, topk_groups=1,
              topk=2, score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=640,
              inter_shared=384, act_dtype="bf16", w_dtype="fp8", router_dtype="bf16",
              seed=12008),
    MoEConfig("s9_mini_bf16_large_experts", T=1200, dim=384, E=8, n_groups=2, topk_groups=1,
              topk=4, score_func="sigmoid", route_scale=2.5, bias_range=0.05, inter=320,
              inter_shared=192, act_dtype="bf16", w_dtype="bf16", router_dtype="bf16",
              seed=12009),
]


def config_by_name(name: str) -> MoEConfig:
    for c in CONFIGS + SMALL_CONFIGS:
        if c.name == name or c.name.split("_")[0] == name:
            return c
    raise KeyError(name)


# ---------------------------------------------------------------------------
# storage formats (input encodings, not layer arithmetic)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Finite inputs."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_e4m3_codes(v: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes, round to nearest even, saturating to +-448.

    Bit-level: normal range by rounding the fp32 mantissa to 3 bits, the
    subnormal range (|v| < 2^-6, spacing 2^-9) by rounding |v|*512 to an
    integer.
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    u = v.view(np.uint32)
    sign = ((u >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint8)
    mag = u & np.uint32(0x7FFFFFFF)
    lsb = (mag >> np.uint32(20)) & np.uint32(1)
    r = (mag + np.uint32(0x7FFFF) + lsb) >> np.uint32(20)          # (exp32 << 3) | mant3
    normal = r.astype(np.int64) - (120 << 3)                        # rebias exponent 127 -> 7
    sub = np.rint(np.abs(v).astype(np.float64) * 512.0).astype(np.int64)  # half-even
    code = np.where(mag < np.uint32(0x3C800000), sub, normal)       # 2^-6 = 0x3C800000
    code = np.clip(code, 0, 0x7E).astype(np.uint8)
    return code | sign


def quantize_weight_blocks(w: np.ndarray):
    """[N, K] fp32 -> (codes uint8 [N, K], scales fp32 [ceil(N/128), K/128]).

    scale = amax/448 over each 128x128 block (1.0 for an all-zero block);
    code = e4m3(w / scale).
    """
    N, K = w.shape
    nb, kb = -(-N // FP8_BLOCK), K // FP8_BLOCK
    pad = nb * FP8_BLOCK - N
    wp = np.pad(w, ((0, pad), (0, 0))) if pad else w
    blk = wp.reshape(nb, FP8_BLOCK, kb, FP8_BLOCK)
    amax = np.abs(blk).max(axis=(1, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = f32_to_e4m3_codes(blk / scale[:, None, :, None])
    return q.reshape(nb * FP8_BLOCK, K)[:N].copy(), scale


# ---------------------------------------------------------------------------
# drawing
# ---------------------------------------------------------------------------

def _rng(cfg: MoEConfig, tag: int, idx: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([cfg.seed, tag, idx]))


def _encode(a: np.ndarray, dt: str):
    if dt == "f32":
        return a.astype(np.float32)
    if dt == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(dt)


def _normal(cfg, tag, idx, shape, fan_in):
    g = _rng(cfg, tag, idx)
    a = g.standard_normal(shape, dtype=np.float32)
    a *= np.float32(1.0 / np.sqrt(fan_in))
    return a


@dataclass
class ExpertWeights:
    """One SwiGLU weight set in storage format.

    w1, w3: [inter, dim]; w2: [dim, inter] (all [out, in]).
    For "f32" the arrays are float32, for "bf16" uint16 bit patterns, for
    "fp8" uint8 e4m3fn codes with fp32 block scales in w1_s [inter/128, dim/128],
    w3_s likewise and w2_s [dim/128, inter/128]; otherwise the *_s are None.
    """

    w1: np.ndarray
    w3: np.ndarray
    w2: np.ndarray
    w1_s: Optional[np.ndarray] = None
    w3_s: Optional[np.ndarray] = None
    w2_s: Optional[np.ndarray] = None


def draw_expert(cfg: MoEConfig, e: int, shared: bool = False) -> ExpertWeights:
    """Weights of routed expert e (or of the shared expert)."""
    inter = cfg.inter_shared if shared else cfg.inter
    t1, t3, t2 = (TAG_WS1, TAG_WS3, TAG_WS2) if shared else (TAG_W1, TAG_W3, TAG_W2)
    a1 = _normal(cfg, t1, e, (inter, cfg.dim), cfg.dim)
    a3 = _normal(cfg, t3, e, (inter, cfg.dim), cfg.dim)
    a2 = _normal(cfg, t2, e, (cfg.dim, inter), inter)
    if cfg.w_dtype == "fp8":
        q1, s1 = quantize_weight_blocks(a1)
        q3, s3 = quantize_weight_blocks(a3)
        q2, s2 = quantize_weight_blocks(a2)
        return ExpertWeights(q1, q3, q2, s1, s3, s2)
    return ExpertWeights(_encode(a1, cfg.w_dtype), _encode(a3, cfg.w_dtype),
                         _encode(a2, cfg.w_dtype))


@dataclass
class Layer:
    """All inputs of one layer forward, in storage format.

    x [T, dim]; wr [E, dim]; bias [E] fp32 or None; w1/w3 [E, inter, dim] and
    w2 [E, dim, inter] stacked over experts (with *_s block scales for fp8);
    shared: ExpertWeights or None.
    """

    cfg: MoEConfig
    x: np.ndarray
    wr: np.ndarray
    bias: Optional[np.ndarray]
    hot: np.ndarray
    w1: np.ndarray
    w3: np.ndarray
    w2: np.ndarray
    w1_s: Optional[np.ndarray] = None
    w3_s: Optional[np.ndarray] = None
    w2_s: Optional[np.ndarray] = None
    shared: Optional[ExpertWeights] = None
    extra: dict = field(default_factory=dict)

    def expert(self, e: int) -> ExpertWeights:
        if self.w1_s is None:
            return ExpertWeights(self.w1[e], self.w3[e], self.w2[e])
        return ExpertWeights(self.w1[e], self.w3[e], self.w2[e],
                             self.w1_s[e], self.w3_s[e], self.w2_s[e])


def draw_router(cfg: MoEConfig):
    """(wr, bias, hot): router weight in storage format, fp32 bias or None, hot ids."""
    wr = _normal(cfg, TAG_WR, 0, (cfg.E, cfg.dim), cfg.dim)
    wr = _encode(wr, cfg.router_dtype)
    hot = np.zeros(0, dtype=np.int64)
    if cfg.hot_experts:
        hot = np.sort(_rng(cfg, TAG_HOT).choice(cfg.E, cfg.hot_experts, replace=False))
        if cfg.router_dtype == "bf16":
            v = bf16_bits_to_f32(wr[hot]) * np.float32(cfg.hot_scale)  # exact (power of two)
            wr[hot] = f32_to_bf16_bits(v)
        else:
            wr[hot] *= np.float32(cfg.hot_scale)
    bias = None
    if cfg.bias_range is not None:
        bias = _rng(cfg, TAG_BIAS).uniform(-cfg.bias_range, cfg.bias_range, cfg.E).astype(np.float32)
    return wr, bias, hot


def draw_x(cfg: MoEConfig) -> np.ndarray:
    return _encode(_rng(cfg, TAG_X).standard_normal((cfg.T, cfg.dim), dtype=np.float32),
                   cfg.act_dtype)


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_layer(cfg: MoEConfig, threads: Optional[int] = None, sink=None) -> Layer:
    """Draw every input of cfg.

    Experts are drawn in parallel threads (numpy releases the GIL while
    filling).  ``sink(e, ExpertWeights)`` is called for each routed expert
    (e.g. to copy it to the device) before it is stored in the stacked arrays.
    """
    threads = threads or default_threads()
    wr, bias, hot = draw_router(cfg)
    x = draw_x(cfg)
    E, inter, dim = cfg.E, cfg.inter, cfg.dim
    if cfg.w_dtype == "fp8":
        st = np.uint8
    elif cfg.w_dtype == "bf16":
        st = np.uint16
    else:
        st = np.float32
    w1 = np.empty((E, inter, dim), st)
    w3 = np.empty((E, inter, dim), st)
    w2 = np.empty((E, dim, inter), st)
    scales = None
    if cfg.w_dtype == "fp8":
        nbi, nbd = -(-inter // FP8_BLOCK), dim // FP8_BLOCK
        scales = (np.empty((E, nbi, nbd), np.float32), np.empty((E, nbi, nbd), np.float32),
                  np.empty((E, -(-dim // FP8_BLOCK), inter // FP8_BLOCK), np.float32))

    def one(e):
        ew = draw_expert(cfg, e)
        w1[e], w3[e], w2[e] = ew.w1, ew.w3, ew.w2
        if scales is not None:
            scales[0][e], scales[1][e], scales[2][e] = ew.w1_s, ew.w3_s, ew.w2_s
        if sink is not None:
            sink(e, ew)

    if threads == 1 or E == 1:
        for e in range(E):
            one(e)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(E)))
    shared = draw_expert(cfg, 0, shared=True) if cfg.inter_shared else None
    layer = Layer(cfg, x, wr, bias, hot, w1, w3, w2, shared=shared)
    if scales is not None:
        layer.w1_s, layer.w3_s, layer.w2_s = scales
    return layer
