"""Latent-MoE layer forward for AMD Instinct MI355X (gfx950).

The compute lives in liblmoe.so (hand-written HIP kernels behind the C ABI of
include/lmoe.h); `binding` exposes that ABI to Python and `layer` sequences it.
"""
from . import binding
from .binding import LmoeError
from .layer import LatentMoELayer, LayerShape, NativeLayer, StepTimer

__all__ = ["binding", "LmoeError", "LatentMoELayer", "LayerShape", "NativeLayer", "StepTimer"]
