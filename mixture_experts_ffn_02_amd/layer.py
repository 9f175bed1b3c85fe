"""Python face of libmoe.so: one MoE FFN layer whose weights live in HBM.

PyTorch supplies device memory and the current HIP stream; every computation
is a call into the C ABI (include/moe.h), whose kernels do all the work.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import _native as N
from .inputs import LayerConfig


def to_device(a: Optional[np.ndarray], device="cuda") -> Optional[torch.Tensor]:
    """Host array (fp32, or bf16 bit patterns as uint16) -> contiguous device tensor."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device).contiguous()


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array (bf16 comes back as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return N.MOE_BF16
    if t.dtype == torch.float32:
        return N.MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


class Timing:
    """Per-phase hipEvent timing of moe_forward_ex; `phases` (names from
    N.PHASES) limits the events to those phases' boundaries."""

    def __init__(self, phases: Optional[Sequence[str]] = None):
        self.lib = N.load()
        h = ctypes.c_void_p()
        N.check(self.lib.moe_timing_create(ctypes.byref(h)), "moe_timing_create")
        self.h = h
        if phases is not None:
            mask = 0
            for p in phases:
                mask |= 1 << N.PHASES.index(p)
            N.check(self.lib.moe_timing_select(self.h, mask), "moe_timing_select")

    def read(self) -> Dict[str, float]:
        """Milliseconds per phase; phases not timed are left out."""
        ms = (ctypes.c_float * N.MOE_N_PHASES)()
        N.check(self.lib.moe_timing_read(self.h, ms), "moe_timing_read")
        return {name: float(ms[i]) for i, name in enumerate(N.PHASES) if ms[i] >= 0.0}

    def close(self):
        if self.h:
            self.lib.moe_timing_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class MoELayer:
    """Weights of one layer on the GPU plus its C description."""

    def __init__(self, cfg: LayerConfig, tensors: Dict[str, Optional[torch.Tensor]]):
        self.lib = N.load()
        self.cfg = cfg
        self.t = tensors
        c = N.MoeLayerC()
        c.d_model, c.d_ff, c.n_experts, c.top_k = cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k
        c.score = N.MOE_SIGMOID if cfg.score == "sigmoid" else N.MOE_SOFTMAX
        c.renorm = int(bool(cfg.renorm))
        c.dtype = N.MOE_BF16 if cfg.dtype == "bf16" else N.MOE_F32
        c.d_ff_shared = cfg.d_ff_s
        c.bias_on_logits = int(bool(cfg.bias_on_logits))
        for name in ("w_router", "sel_bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
            tt = tensors.get(name)
            setattr(c, name, None if tt is None else tt.data_ptr())
        self.c = c
        self._ws: Optional[torch.Tensor] = None
        self._bws: Optional[torch.Tensor] = None
        self.device = tensors["w_router"].device

    @classmethod
    def from_host(cls, cfg: LayerConfig, inputs: Dict[str, Optional[np.ndarray]], device="cuda") -> "MoELayer":
        names = ("w_router", "sel_bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
        return cls(cfg, {n: to_device(inputs.get(n), device) for n in names})

    # -------------------------------------------------------------- helpers
    def workspace_bytes(self, T: int) -> int:
        n = ctypes.c_size_t()
        N.check(self.lib.moe_workspace_size(ctypes.byref(self.c), T, ctypes.byref(n)), "moe_workspace_size")
        return n.value

    def workspace(self, T: int) -> torch.Tensor:
        need = max(1, self.workspace_bytes(T))
        if self._ws is None or self._ws.numel() < need:
            self._ws = None
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def _opts(self, T: int, noise: Optional[torch.Tensor], metrics: bool):
        """moe_route_opts for one call, and the metrics tensor it fills."""
        if noise is None and not metrics:
            return None, None
        if noise is not None and (noise.shape != (T, self.cfg.n_experts) or noise.dtype != torch.float32
                                  or not noise.is_contiguous()):
            raise ValueError(f"noise must be contiguous fp32 [T, {self.cfg.n_experts}]")
        m = torch.empty(N.MOE_N_METRICS, dtype=torch.float64, device=self.device) if metrics else None
        o = N.MoeRouteOptsC()
        o.sel_noise = None if noise is None else noise.data_ptr()
        o.metrics = None if m is None else m.data_ptr()
        return o, m

    def _check_x(self, x: torch.Tensor) -> int:
        if x.dim() != 2 or x.shape[1] != self.cfg.d_model or not x.is_contiguous():
            raise ValueError(f"x must be contiguous [T, {self.cfg.d_model}]")
        if _dtype_code(x) != self.c.dtype:
            raise TypeError("x dtype does not match the layer dtype")
        return x.shape[0]

    # ---------------------------------------------------------- entry points
    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None, want_routing: bool = True,
                timing: Optional[Timing] = None, noise: Optional[torch.Tensor] = None,
                metrics: bool = False) -> Dict[str, torch.Tensor]:
        """y = the layer applied to x; with want_routing also idx, w and counts;
        noise [T, E] fp32 is added to the selection values; metrics: the
        router losses and health metrics (fp64 [6], order of METRICS)."""
        T = self._check_x(x)
        k, E, d = self.cfg.top_k, self.cfg.n_experts, self.cfg.d_model
        dev = x.device
        if y is None:
            y = torch.empty((T, d), dtype=torch.float32, device=dev)
        out = {"y": y}
        idx = w = counts = None
        if want_routing:
            idx = torch.empty((T, k), dtype=torch.int32, device=dev)
            w = torch.empty((T, k), dtype=torch.float32, device=dev)
            counts = torch.empty((E,), dtype=torch.int32, device=dev)
            out.update(idx=idx, w=w, counts=counts)
        ws = self.workspace(T)
        opts, m = self._opts(T, noise, metrics)
        if opts is None and timing is None:
            N.check(self.lib.moe_forward(ctypes.byref(self.c), _p(x), T, _p(y), _p(idx), _p(w), _p(counts), _p(ws),
                                         ws.numel(), _stream()), "moe_forward")
        else:
            N.check(self.lib.moe_forward_ex(ctypes.byref(self.c), _p(x), T, None if opts is None else ctypes.byref(opts),
                                            _p(y), _p(idx), _p(w), _p(counts), _p(ws), ws.numel(), _stream(),
                                            None if timing is None else timing.h), "moe_forward_ex")
        if m is not None:
            out["metrics"] = m
        return out

    def route(self, x: torch.Tensor, noise: Optional[torch.Tensor] = None,
              metrics: bool = False) -> Dict[str, torch.Tensor]:
        T = self._check_x(x)
        k, E = self.cfg.top_k, self.cfg.n_experts
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
        counts = torch.empty((E,), dtype=torch.int32, device=x.device)
        ws = self.workspace(T)
        opts, m = self._opts(T, noise, metrics)
        if opts is None:
            N.check(self.lib.moe_route(ctypes.byref(self.c), _p(x), T, _p(idx), _p(w), _p(counts), _p(ws),
                                       ws.numel(), _stream()), "moe_route")
        else:
            N.check(self.lib.moe_route_ex(ctypes.byref(self.c), _p(x), T, ctypes.byref(opts), _p(idx), _p(w),
                                          _p(counts), _p(ws), ws.numel(), _stream()), "moe_route_ex")
        out = {"idx": idx, "w": w, "counts": counts}
        if m is not None:
            out["metrics"] = m
        return out

    def bias_update(self, counts: torch.Tensor, rate: float) -> torch.Tensor:
        """One balance-controller step on this layer's selection bias, in place."""
        b = self.t.get("sel_bias")
        if b is None:
            raise ValueError("the layer has no selection bias")
        bias_update(counts, b, rate)
        return b

    def backward_workspace_bytes(self, T: int) -> int:
        n = ctypes.c_size_t()
        N.check(self.lib.moe_backward_workspace_size(ctypes.byref(self.c), T, ctypes.byref(n)),
                "moe_backward_workspace_size")
        return n.value

    def backward(self, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, z_loss_coef: float = 0.0,
                 aux_loss_coef: float = 0.0) -> Dict[str, torch.Tensor]:
        """moe_backward: fp32 gradients of x, the router, the expert weights
        (and the shared expert's) and the combine weights, for the routing
        (idx, w) of the forward pass and dy = dL/dy [T, d] fp32."""
        T = self._check_x(x)
        c = self.cfg
        E, k, d, f, fs = c.n_experts, c.top_k, c.d_model, c.d_ff, c.d_ff_s
        dev = x.device
        for name, t, shape, dt in (("idx", idx, (T, k), torch.int32), ("w", w, (T, k), torch.float32),
                                   ("dy", dy, (T, d), torch.float32)):
            if t.shape != shape or t.dtype != dt or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous {dt} {shape}")
        z = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
        g = {"dx": z(T, d), "dw_router": z(E, d), "dw_gate": z(E, f, d), "dw_up": z(E, f, d), "dw_down": z(E, d, f),
             "d_topk_w": z(T, k)}
        if fs:
            g.update(dws_gate=z(fs, d), dws_up=z(fs, d), dws_down=z(d, fs))
        gc = N.MoeGradsC(*[None if g.get(n) is None else g[n].data_ptr() for n, _ in N.MoeGradsC._fields_])
        need = max(1, self.backward_workspace_bytes(T))
        if self._bws is None or self._bws.numel() < need:
            self._bws = None
            self._bws = torch.empty(need, dtype=torch.uint8, device=dev)
        ws = self._bws
        N.check(self.lib.moe_backward(ctypes.byref(self.c), _p(x), T, _p(idx), _p(w), _p(dy), float(z_loss_coef),
                                      float(aux_loss_coef), ctypes.byref(gc), _p(ws), ws.numel(), _stream()),
                "moe_backward")
        return g

    def permute(self, x: torch.Tensor, idx: torch.Tensor, with_rows: bool = True) -> Dict[str, torch.Tensor]:
        T = self._check_x(x)
        k, E, d = self.cfg.top_k, self.cfg.n_experts, self.cfg.d_model
        if idx.shape != (T, k) or idx.dtype != torch.int32 or not idx.is_contiguous():
            raise ValueError("idx must be contiguous int32 [T, k]")
        x_perm = torch.empty((T * k, d), dtype=x.dtype, device=x.device) if with_rows else None
        offsets = torch.empty((E + 1,), dtype=torch.int32, device=x.device)
        row_of = torch.empty((T, k), dtype=torch.int32, device=x.device)
        ws = self.workspace(T)
        N.check(self.lib.moe_permute(ctypes.byref(self.c), _p(x), T, _p(idx), _p(x_perm), _p(offsets), _p(row_of),
                                     _p(ws), ws.numel(), _stream()), "moe_permute")
        return {"x_perm": x_perm, "offsets": offsets, "row_of": row_of}

    def combine(self, y_perm: torch.Tensor, row_of: torch.Tensor, w: torch.Tensor,
                y_shared: Optional[torch.Tensor] = None) -> torch.Tensor:
        T = row_of.shape[0]
        y = torch.empty((T, self.cfg.d_model), dtype=torch.float32, device=y_perm.device)
        N.check(self.lib.moe_combine(ctypes.byref(self.c), T, _p(y_perm), _p(row_of), _p(w), _p(y_shared), _p(y),
                                     _stream()), "moe_combine")
        return y


def bias_update(counts: torch.Tensor, bias: torch.Tensor, rate: float) -> None:
    """moe_bias_update: bias [E] fp32 updated in place from counts [E] int32."""
    if counts.dtype != torch.int32 or bias.dtype != torch.float32 or counts.numel() != bias.numel():
        raise ValueError("counts must be int32 [E] and bias fp32 [E]")
    if not (counts.is_contiguous() and bias.is_contiguous()):
        raise ValueError("counts and bias must be contiguous")
    N.check(N.load().moe_bias_update(bias.numel(), _p(counts), float(rate), _p(bias), _stream()), "moe_bias_update")


def grouped_swiglu(a: torch.Tensor, offsets: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
                   w_down: torch.Tensor) -> torch.Tensor:
    """SwiGLU experts over row groups: out [rows, d_in] fp32 (moe_grouped_swiglu)."""
    lib = N.load()
    dt = _dtype_code(a)
    rows, d_in = a.shape
    G, d_ff, _ = w_gate.shape
    n = ctypes.c_size_t()
    N.check(lib.moe_grouped_swiglu_workspace_size(dt, G, d_in, d_ff, rows, ctypes.byref(n)),
            "moe_grouped_swiglu_workspace_size")
    ws = torch.empty(max(1, n.value), dtype=torch.uint8, device=a.device)
    out = torch.empty((rows, d_in), dtype=torch.float32, device=a.device)
    N.check(lib.moe_grouped_swiglu(dt, G, d_in, d_ff, rows, _p(a), _p(offsets), _p(w_gate), _p(w_up), _p(w_down),
                                   _p(out), _p(ws), ws.numel(), _stream()), "moe_grouped_swiglu")
    return out
