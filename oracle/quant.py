"""Oracle for the FP8 fake-quantizers (dispatch rows and combine rows).

Test infrastructure only (see the package docstring).

Sources:
* "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM Mega-MoE",
  PR summary and "How it works": the dispatch quantizer fake-quantizes the
  experts' input tokens before the FP8 staging; the combine quantizer
  fake-quantizes the router-weighted per-(token, slot) BF16 rows; serving
  needs a calibrated (max) or constant global combine scale, since the rows
  a rank quantizes were produced on every expert rank, not just its own;
  "Testing": the calibrated
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

from .numerics import bf16_bits_to_f32, qdq_e4m3fn, e4m3fn_round, E4M3FN_MAX


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


def quantize_weight_blocks(w_bits, block: int = 128):
    """FP8 weights with one scale per ``block x block`` tile of a bfloat16
    matrix ``[N, K]`` (both multiples of ``block``): the weight half of the
    real FP8 grouped GEMM ("next" after the fake-quant units: weights in
    E4M3 with 128x128 block scales).

    ``s = fl32(amax / 448)`` per tile (``amax == 0`` gives ``s = 0``), element
    ``q = e4m3(clamp(fl32(w / s), +-448))``.  Returns ``(q float64 [N, K]`` —
    the E4M3 values themselves — ``, s float32 [N/block, K/block],
    dequantized bf16 bits [N, K])`` where the dequantized weight is
    ``bf16(fl32(q * s))``: the FP8 fake-quant of ``w`` with the tile's scale,
    which is exactly what a GEMM on the FP8 weights multiplies.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    if N % block or K % block:
        raise ValueError("both dimensions must be multiples of the block size")
    w = bf16_bits_to_f32(w_bits).reshape(N // block, block, K // block, block)
    amax = np.abs(w).max(axis=(1, 3))                                  # exact, float32
    s = (amax / np.float32(E4M3FN_MAX)).astype(np.float32)             # IEEE division
    sb = s[:, None, :, None]
    safe = np.where(sb > 0, sb, np.float32(1))
    r = np.clip((w / safe).astype(np.float32), -E4M3FN_MAX, E4M3FN_MAX)
    q = np.where(sb > 0, e4m3fn_round(r), 0.0)
    deq = qdq_e4m3fn(w, sb).reshape(N, K)
    return q.reshape(N, K), s, deq
