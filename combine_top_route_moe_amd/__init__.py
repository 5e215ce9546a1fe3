"""MI355X-native (gfx950) MoE-layer hot path.

route -> (dispatch FP8 fake-quant) -> permute -> grouped SwiGLU FFN on BF16
MFMA -> (combine-row FP8 fake-quant) -> ordered combine, each stage a
hand-written HIP kernel in ``libmoe.so`` behind the C ABI of
``include/moe.h``.  ``ops`` binds every entry point by name (ctypes; torch
only supplies device memory and streams) and ``layer.MoELayer`` owns the
buffers of one layer and enqueues the stages in order.
"""

from . import ops
from ._lib import load, MoEError
from .layer import MoELayer

__all__ = ["ops", "load", "MoEError", "MoELayer"]
