"""CPU oracle for the forward pass of one MoE FFN layer (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It loads ``liboracle.so``, built from ``oracle.c`` by ``build()``
with gcc (``-O3 -ffp-contract=off``, OpenMP, no fast-math), and wraps it for
numpy arrays. It never touches the HIP path and the HIP path never touches it.

Precision: the router runs in fp32 with a fixed fma order (the pages force the
router to fp32: moe-200m-qwen3-100b README, "Per-layer numerics"); the expert
MLPs and the combine run in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O3", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-mavx2", "-mfma",
          "-fopenmp", "-fPIC", "-shared"]

DT = {"f32": 0, "bf16": 1}
SCORE = {"softmax": 0, "sigmoid": 1}

_lib = None


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    """Compile the oracle with gcc; returns the library path."""
    cmd = ["gcc", *CFLAGS, *extra, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def load(path: str = LIB) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_cexpf.restype = ctypes.c_float
    lib.oracle_cexpf.argtypes = [ctypes.c_float]
    lib.oracle_cexpf_array.argtypes = [vp, vp, i64]
    lib.oracle_logits.argtypes = [i32, vp, i64, i32, vp, i32, vp]
    lib.oracle_route.restype = i32
    lib.oracle_route.argtypes = [i32, vp, i64, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.oracle_route_ex.restype = i32
    lib.oracle_route_ex.argtypes = [i32, vp, i64, i32, vp, vp, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.oracle_router_metrics.argtypes = [vp, vp, i64, i32, i32, i32, vp]
    lib.oracle_bias_update.argtypes = [vp, i32, ctypes.c_float, vp]
    lib.oracle_backward.restype = i32
    lib.oracle_backward.argtypes = [i32, vp, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                    vp, vp, vp, ctypes.c_double, ctypes.c_double] + [vp] * 9
    lib.oracle_dispatch.restype = i32
    lib.oracle_dispatch.argtypes = [i64, i32, i32, vp, vp, vp, vp]
    lib.oracle_experts.restype = i32
    lib.oracle_experts.argtypes = [i32, i32, i32, vp, i64, vp, vp, i32, vp, vp, vp, vp]
    lib.oracle_experts_abs.restype = i32
    lib.oracle_experts_abs.argtypes = [i32, i32, i32, vp, i64, vp, vp, i32, vp, vp, vp, vp]
    lib.oracle_combine.restype = i32
    lib.oracle_combine.argtypes = [i32, i32, i32, i32, vp, i64, vp, i32, vp, vp, i32,
                                   vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_num_threads.restype = i32
    return lib


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = load()
    return _lib


def _dt(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return DT["bf16"]
    if x.dtype == np.float32:
        return DT["f32"]
    raise TypeError(f"unsupported dtype {x.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
# wrappers
# ---------------------------------------------------------------------------

def cexpf(a: np.ndarray, L=None) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty_like(a)
    (L or lib()).oracle_cexpf_array(_p(a), _p(out), a.size)
    return out


def logits(x: np.ndarray, w_router: np.ndarray, L=None) -> np.ndarray:
    x = _c(x)
    wr = _c(w_router, np.float32)
    T, d = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float32)
    (L or lib()).oracle_logits(_dt(x), _p(x), T, d, _p(wr), E, _p(out))
    return out


def route(x, w_router, sel_bias, top_k, score="softmax", renorm=True, L=None, bias_on_logits=False,
          noise=None) -> Dict[str, np.ndarray]:
    """fp32 router: idx [T,k] int32, w [T,k] fp32, counts [E] int32, logits [T,E].
    bias_on_logits: the bias enters the logit instead of the score; noise
    [T,E] fp32 is added to the selection value (training-time exploration)."""
    x = _c(x)
    wr = _c(w_router, np.float32)
    b = _c(sel_bias, np.float32)
    nz = _c(noise, np.float32)
    T, d = x.shape
    E = wr.shape[0]
    idx = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    counts = np.empty(E, np.int32)
    lg = np.empty((T, E), np.float32)
    rc = (L or lib()).oracle_route_ex(_dt(x), _p(x), T, d, _p(wr), _p(b), int(bool(bias_on_logits)), _p(nz), E,
                                      top_k, SCORE[score], int(bool(renorm)), _p(idx), _p(w), _p(counts), _p(lg))
    if rc != 0:
        raise ValueError("oracle_route: bad arguments")
    return {"idx": idx, "w": w, "counts": counts, "logits": lg}


METRICS = ("z_loss", "aux_loss", "cv", "entropy_bits", "load_max_ratio", "unused_frac")


def router_metrics(logits, idx, score="softmax", L=None) -> np.ndarray:
    """fp64 router losses and health metrics, in the order of METRICS."""
    lg = _c(logits, np.float32)
    idx = _c(idx, np.int32)
    T, E = lg.shape
    out = np.zeros(len(METRICS), np.float64)
    (L or lib()).oracle_router_metrics(_p(lg), _p(idx), T, E, idx.shape[1], SCORE[score], _p(out))
    return out


def bias_update(counts, bias, rate, L=None) -> np.ndarray:
    """One step of the aux-loss-free balance controller; returns the new bias."""
    c = _c(counts, np.int32)
    b = np.array(bias, dtype=np.float32, copy=True)
    (L or lib()).oracle_bias_update(_p(c), c.size, float(rate), _p(b))
    return b


def dispatch(idx: np.ndarray, n_experts: int, L=None) -> Dict[str, np.ndarray]:
    """counts [E], offsets [E+1], row_of [T,k] (stable by token)."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(n_experts, np.int32)
    offsets = np.empty(n_experts + 1, np.int32)
    row_of = np.empty((T, k), np.int32)
    rc = (L or lib()).oracle_dispatch(T, n_experts, k, _p(idx), _p(counts), _p(offsets), _p(row_of))
    if rc != 0:
        raise ValueError("oracle_dispatch: expert index out of range")
    return {"counts": counts, "offsets": offsets, "row_of": row_of}


def experts(x, pair_row, pair_expert, w_gate, w_up, w_down, L=None, absolute=False) -> np.ndarray:
    """fp64 SwiGLU expert outputs for (row, expert) pairs: [n_pairs, d].
    absolute=True gives the magnitude envelope sum_f |W_down| |h_f| instead."""
    x = _c(x)
    pr = _c(pair_row, np.int64)
    pe = _c(pair_expert, np.int32)
    wg, wu, wd = _c(w_gate), _c(w_up), _c(w_down)
    if wg.ndim == 2:
        wg, wu, wd = wg[None], wu[None], wd[None]
    E, d_ff, d = wg.shape
    out = np.zeros((pr.size, d), np.float64)
    fn = (L or lib()).oracle_experts_abs if absolute else (L or lib()).oracle_experts
    rc = fn(_dt(x), d, d_ff, _p(x), pr.size, _p(pr), _p(pe), E, _p(wg), _p(wu), _p(wd), _p(out))
    if rc != 0:
        raise ValueError("oracle_experts: expert index out of range")
    return out


def combine(x, tokens, idx, w, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None, L=None) -> np.ndarray:
    """fp64 layer output for the listed tokens: [n_tok, d]."""
    x = _c(x)
    tokens = _c(tokens, np.int64)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    wg, wu, wd = _c(w_gate), _c(w_up), _c(w_down)
    sg, su, sd = _c(ws_gate), _c(ws_up), _c(ws_down)
    E, d_ff, d = wg.shape
    k = idx.shape[1]
    d_ff_s = sg.shape[0] if sg is not None else 0
    y = np.zeros((tokens.size, d), np.float64)
    rc = (L or lib()).oracle_combine(_dt(x), d, d_ff, d_ff_s, _p(x), tokens.size, _p(tokens), k, _p(idx), _p(w), E,
                                     _p(wg), _p(wu), _p(wd), _p(sg), _p(su), _p(sd), _p(y))
    if rc != 0:
        raise ValueError("oracle_combine: bad arguments")
    return y


def forward(inputs: Dict[str, np.ndarray], top_k: int, score: str, renorm: bool = True,
            tokens: Optional[np.ndarray] = None, L=None, bias_on_logits: bool = False,
            noise: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The whole layer: routing for every token, dispatch order, and the fp64
    output y for ``tokens`` (all tokens when None)."""
    x = inputs["x"]
    r = route(x, inputs["w_router"], inputs.get("sel_bias"), top_k, score, renorm, L=L,
              bias_on_logits=bias_on_logits, noise=noise)
    E = inputs["w_router"].shape[0]
    dsp = dispatch(r["idx"], E, L=L)
    if tokens is None:
        tokens = np.arange(x.shape[0], dtype=np.int64)
    y = combine(x, tokens, r["idx"], r["w"], inputs["w_gate"], inputs["w_up"], inputs["w_down"],
                inputs.get("ws_gate"), inputs.get("ws_up"), inputs.get("ws_down"), L=L)
    out = dict(r)
    out.update(offsets=dsp["offsets"], row_of=dsp["row_of"], y=y, tokens=np.asarray(tokens, np.int64))
    return out


def backward(inputs: Dict[str, np.ndarray], idx, w, dy, score: str, renorm: bool = True, z_coef: float = 0.0,
             aux_coef: float = 0.0, L=None) -> Dict[str, np.ndarray]:
    """fp64 gradients of the layer for a given routing (idx, w from the forward
    pass) and output gradient dy [T, d]: dx, dw_router, dw_gate, dw_up,
    dw_down, the shared expert's (or None) and d_topk_w (the combine weights)."""
    x = _c(inputs["x"])
    T, d = x.shape
    wr = _c(inputs["w_router"], np.float32)
    wg, wu, wd = _c(inputs["w_gate"]), _c(inputs["w_up"]), _c(inputs["w_down"])
    E, d_ff, _ = wg.shape
    sg, su, sd = _c(inputs.get("ws_gate")), _c(inputs.get("ws_up")), _c(inputs.get("ws_down"))
    d_ff_s = 0 if sg is None else sg.shape[0]
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    dy = _c(dy, np.float32)
    k = idx.shape[1]
    out = {
        "dx": np.zeros((T, d)), "dw_router": np.zeros((E, d)), "dw_gate": np.zeros((E, d_ff, d)),
        "dw_up": np.zeros((E, d_ff, d)), "dw_down": np.zeros((E, d, d_ff)),
        "dws_gate": None if sg is None else np.zeros((d_ff_s, d)),
        "dws_up": None if sg is None else np.zeros((d_ff_s, d)),
        "dws_down": None if sg is None else np.zeros((d, d_ff_s)),
        "d_topk_w": np.zeros((T, k)),
    }
    rc = (L or lib()).oracle_backward(
        _dt(x), _p(x), T, d, E, k, d_ff, d_ff_s, _p(wr), _p(wg), _p(wu), _p(wd), _p(sg), _p(su), _p(sd),
        SCORE[score], int(bool(renorm)), _p(idx), _p(w), _p(dy), float(z_coef), float(aux_coef),
        *[_p(out[n]) for n in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down",
                               "d_topk_w")])
    if rc != 0:
        raise ValueError("oracle_backward: expert index out of range")
    return out
