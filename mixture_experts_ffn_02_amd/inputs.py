"""Seeded synthetic inputs for one Mixture-of-Experts FFN layer.

This module holds shapes, seeds and random draws only. It contains none of the
layer's arithmetic (no gate product, no scores, no top-k, no SwiGLU, no
combine), so both the HIP path and the CPU oracle can take their inputs from it
without sharing any of the method.

Generator recipe
----------------
* numpy ``default_rng([seed, tensor_id, part])`` (PCG64). Every tensor, and
  every expert of a stacked tensor, has its own stream, so generation is
  chunkable and runs on several threads with identical results.
* Values are drawn as fp32 normals (``standard_normal(dtype=float32)``) and
  multiplied by an fp32 standard deviation. For bf16 layers the fp32 values
  are rounded to bf16 with round-to-nearest-even by bit arithmetic and kept as
  ``uint16`` bit patterns. The router weight and the selection bias stay fp32
  in every layer (the router runs in fp32: moe-200m-qwen3-100b README,
  "Per-layer numerics").
* "N(0, s)" means standard deviation s. ``std=None`` means 1/sqrt(fan_in),
  with fan_in = d_model for the router, gate and up weights and d_ff for the
  down weight.
* Expert weights are stacked ``[E, out, in]`` (SpecForge PR #930, "Why FSDP is
  enough here"): gate and up ``[E, d_ff, d_model]``, down ``[E, d_model, d_ff]``.
* Skewed load ("Zipf-like, s over experts"): feature 0 of every token is fixed
  to 1.0 and ``W_r[e, 0] = -s * ln(e + 1)``. Feature 0 then adds a per-expert
  logit offset, so the expected softmax mass of expert e is proportional to
  (e+1)^-s without any change to the layer itself.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

# Stream ids of the tensors of one layer.
TID_X, TID_WR, TID_BIAS, TID_WG, TID_WU, TID_WD, TID_SG, TID_SU, TID_SD, TID_NOISE = range(10)
X_CHUNK_ROWS = 1024


@dataclass(frozen=True)
class LayerConfig:
    """Shape and recipe of one MoE FFN layer and of its synthetic inputs."""

    name: str
    T: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    dtype: str = "bf16"            # x and expert weights: "f32" or "bf16"
    score: str = "softmax"         # "softmax" over all experts, or "sigmoid"
    renorm: bool = True            # renormalise the top-k combine weights
    shared: bool = False           # one always-on shared SwiGLU expert
    d_ff_shared: int = 0           # 0: same width as a routed expert
    bias_range: float = 0.0        # selection bias ~ U(-r, r); 0: no bias
    bias_on_logits: bool = False   # the bias enters the logit instead of the score
    weight_std: Optional[float] = None  # None: 1/sqrt(fan_in) for every weight
    zipf_s: float = 0.0            # > 0: skew the router towards low expert ids
    seed: int = 0

    @property
    def d_ff_s(self) -> int:
        return (self.d_ff_shared or self.d_ff) if self.shared else 0

    def with_tokens(self, T: int) -> "LayerConfig":
        return replace(self, T=T)

    def gemm_flops(self) -> float:
        """Algorithmic flops of the expert GEMMs (activated experts only)."""
        routed = 6.0 * self.T * self.top_k * self.d_model * self.d_ff
        shared = 6.0 * self.T * self.d_model * self.d_ff_s
        return routed + shared


# The five layers of the hot path. Names describe the layer; sizes follow the
# pages' layers (moe-200m-qwen3-100b README "Resulting architecture" for the
# small sigmoid layer; SpecForge PR #930 "What this adds" for the iso-width
# layer and the Qwen3 recipe).
CONFIGS: Dict[str, LayerConfig] = {
    c.name: c
    for c in (
        LayerConfig("tiny_f32", T=256, d_model=64, n_experts=8, top_k=2, d_ff=128,
                    dtype="f32", score="softmax"),
        LayerConfig("small_sigmoid", T=8192, d_model=640, n_experts=16, top_k=2, d_ff=1024,
                    score="sigmoid", shared=True, bias_range=0.5),
        LayerConfig("qwen3_fine", T=16384, d_model=2048, n_experts=128, top_k=8, d_ff=768,
                    score="softmax", zipf_s=1.1),
        LayerConfig("iso_wide", T=32768, d_model=5120, n_experts=16, top_k=4, d_ff=4352,
                    score="softmax", bias_range=0.1, weight_std=0.02),
        LayerConfig("deepseek_fine", T=65536, d_model=7168, n_experts=256, top_k=8, d_ff=2048,
                    score="sigmoid", shared=True, bias_range=0.1),
    )
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns exactly to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(seed: int, tid: int, part: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, part])
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def _stacked(cfg: LayerConfig, tid: int, n: int, out: int, inp: int, pool) -> np.ndarray:
    std = cfg.weight_std if cfg.weight_std is not None else 1.0 / math.sqrt(inp)
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    w = np.empty((n, out, inp), dtype=dt)

    def one(e):
        w[e] = _encode(_normal(cfg.seed, tid, e, (out, inp), std), cfg.dtype)

    list(pool.map(one, range(n)))
    return w


def make_x(cfg: LayerConfig, T: Optional[int] = None, pool=None) -> np.ndarray:
    """Activations [T, d_model]: N(0,1), chunked in row blocks of 1024 tokens."""
    T = cfg.T if T is None else T
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    x = np.empty((T, cfg.d_model), dtype=dt)
    n_chunks = (T + X_CHUNK_ROWS - 1) // X_CHUNK_ROWS

    def one(c):
        r0 = c * X_CHUNK_ROWS
        r1 = min(T, r0 + X_CHUNK_ROWS)
        a = _normal(cfg.seed, TID_X, c, (X_CHUNK_ROWS, cfg.d_model), 1.0)[: r1 - r0]
        if cfg.zipf_s > 0:
            a[:, 0] = 1.0
        x[r0:r1] = _encode(a, cfg.dtype)

    if pool is None:
        with ThreadPoolExecutor(_threads()) as p:
            list(p.map(one, range(n_chunks)))
    else:
        list(pool.map(one, range(n_chunks)))
    return x


def make_layer(cfg: LayerConfig, T: Optional[int] = None, with_experts: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one layer as host numpy arrays.

    Keys: x, w_router, sel_bias (or None), w_gate, w_up, w_down, and, with a
    shared expert, ws_gate, ws_up, ws_down (else None).
    """
    E, d, f = cfg.n_experts, cfg.d_model, cfg.d_ff
    out: Dict[str, Optional[np.ndarray]] = {}
    with ThreadPoolExecutor(_threads()) as pool:
        out["x"] = make_x(cfg, T, pool)
        wr_std = cfg.weight_std if cfg.weight_std is not None else 1.0 / math.sqrt(d)
        wr = _normal(cfg.seed, TID_WR, 0, (E, d), wr_std)
        if cfg.zipf_s > 0:
            wr[:, 0] = (-cfg.zipf_s * np.log(np.arange(E, dtype=np.float64) + 1.0)).astype(np.float32)
        out["w_router"] = wr
        if cfg.bias_range > 0:
            rng = np.random.default_rng([cfg.seed, TID_BIAS, 0])
            out["sel_bias"] = rng.uniform(-cfg.bias_range, cfg.bias_range, E).astype(np.float32)
        else:
            out["sel_bias"] = None
        if with_experts:
            out["w_gate"] = _stacked(cfg, TID_WG, E, f, d, pool)
            out["w_up"] = _stacked(cfg, TID_WU, E, f, d, pool)
            out["w_down"] = _stacked(cfg, TID_WD, E, d, f, pool)
            if cfg.shared:
                fs = cfg.d_ff_s
                out["ws_gate"] = _stacked(cfg, TID_SG, 1, fs, d, pool)[0]
                out["ws_up"] = _stacked(cfg, TID_SU, 1, fs, d, pool)[0]
                out["ws_down"] = _stacked(cfg, TID_SD, 1, d, fs, pool)[0]
            else:
                out["ws_gate"] = out["ws_up"] = out["ws_down"] = None
    return out


def make_noise(cfg: LayerConfig, std: float, step: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Router exploration noise [T, n_experts] fp32: N(0, std), one stream per step."""
    T = cfg.T if T is None else T
    return _normal(cfg.seed, TID_NOISE, step, (T, cfg.n_experts), std)
