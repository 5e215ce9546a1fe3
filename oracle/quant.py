"""Oracle for the FP8 fake-quantizers (dispatch rows and combine rows).

Test infrastructure only (see the package docstring).

Sources:
* "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM Mega-MoE",
  PR summary and "How it works": the dispatch quantizer fake-quantizes the
  experts' input tokens before the FP8 staging; the combine quantizer
  fake-quantizes the router-weighted per-(token, slot) BF16 rows; serving
  needs a calibrated (max) or constant global combine scale because each
  rank re-quantizes rows from all expert ranks; "Testing": the calibrated
  amax equals the max of what the quantizer saw.
* "[Kernel] DeepEP dispatch-combine kernel integration", review thread on
  the low-latency prepare/finalize: FP8 dispatch with a ``block_shape`` and
  per-block scales sent alongside the tokens.
* The workload descriptions: dispatch blocks are per token and per 128
  channels with scale amax/448; the combine scale is 1/448 of max|row|,
  calibrated once.

Formula (for one block, or one tensor with a given scale):
``s = fl32(amax / 448)``;  ``x' = bf16(fl32(e4m3(clamp(fl32(x / s), +-448)) * s))``;
``amax == 0`` gives an all-(+0) block.
"""

import numpy as np

from .numerics import bf16_bits_to_f32, qdq_e4m3fn, E4M3FN_MAX


def fake_quant_block(x_bits, block: int = 128, row_mask=None):
    """Per-row, per-``block``-channel fake-quant of bfloat16 rows.

    ``x_bits``: uint16 [R, H] with H a multiple of ``block``.  ``row_mask``:
    optional bool [R]; rows where it is False are returned unchanged (padding
    tokens are not quantized).  Returns ``(out_bits uint16 [R,H],
    scales float32 [R, H/block])``; masked rows get scale 0.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, H = x_bits.shape
    if H % block:
        raise ValueError("H must be a multiple of the block size")
    x = bf16_bits_to_f32(x_bits).reshape(R, H // block, block)
    amax = np.abs(x).max(axis=2)                              # exact
    s = (amax / np.float32(E4M3FN_MAX)).astype(np.float32)    # IEEE division
    out = qdq_e4m3fn(x, s[:, :, None]).reshape(R, H)
    if row_mask is not None:
        keep = ~np.asarray(row_mask, dtype=bool)
        out[keep] = x_bits[keep]
        s = s.copy()
        s[keep] = 0
    return out, s.astype(np.float32)


def calibrate_amax(x_bits, row_mask=None) -> np.float32:
    """Max calibration: ``max |x|`` over the (selected) rows, as float32."""
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16))
    if row_mask is not None:
        x = x[np.asarray(row_mask, dtype=bool)]
    if x.size == 0:
        return np.float32(0)
    return np.float32(np.abs(x).max())


def scale_from_amax(amax) -> np.float32:
    """The constant per-tensor scale ``fl32(amax / 448)``."""
    return np.float32(np.float32(amax) / np.float32(E4M3FN_MAX))


def fake_quant_per_tensor(x_bits, scale, row_mask=None):
    """Fake-quant of bfloat16 rows with one constant float32 scale.

    Rows where ``row_mask`` is False (pow2 padding rows, or rows the caller
    does not quantize) are returned unchanged.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    out = qdq_e4m3fn(bf16_bits_to_f32(x_bits), np.float32(scale))
    if row_mask is not None:
        keep = ~np.asarray(row_mask, dtype=bool)
        out[keep] = x_bits[keep]
    return out
