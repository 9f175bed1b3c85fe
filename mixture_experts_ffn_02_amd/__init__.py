"""Forward pass of one Mixture-of-Experts FFN layer on one AMD Instinct MI355X.

The work runs in hand-written HIP kernels for gfx950 behind the C ABI of
``libmoe.so`` (include/moe.h): an fp32 router with a wavefront top-k, a
dispatch into expert-contiguous order, SwiGLU experts as grouped GEMMs on
MFMA, and a gather combine. PyTorch only provides device memory and streams.

Modules:
  inputs  seeded synthetic layers (shapes, seeds, random draws only)
  layer   MoELayer / grouped_swiglu / Timing: the Python face of the C ABI
  build   compiles libmoe.so for gfx950 with hipcc
"""
from .inputs import CONFIGS, LayerConfig  # noqa: F401


def __getattr__(name):
    if name in ("MoELayer", "Timing", "grouped_swiglu", "to_device", "to_host"):
        from . import layer

        return getattr(layer, name)
    raise AttributeError(name)
