"""Oracle for the real FP8 grouped FFN: E4M3 activations and weights with
block scales, the scales applied per 128-wide K-block.  Test
infrastructure only (see the package docstring).

Sources:
* "[Kernel] DeepEP dispatch-combine kernel integration", review thread on
  the low-latency dispatch: the dispatch quantizes the tokens to FP8 and
  hands over the codes together with their block scales, which the
  receiving side uses; review thread on the DeepEP + DeepGEMM test: the
  expert weights carry one scale per ``block_n x block_k`` tile, consumed by
  DeepGEMM's FP8 grouped GEMMs.
* "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM
  Mega-MoE", "How it works": the dispatch quantizer's codes and scales are
  those its fake-quant dequantizes (the fake-quant is this quantizer
  followed by ``bf16(q * s)``).

Readings (also in the design notes):
* activation blocks are 1 x 128 along the reduction dimension, weight tiles
  128 x 128; ``s = fl32(amax / 448)`` and code ``e4m3(clamp(fl32(x / s), +-448))``
  as in the fake-quantizers; an all-zero block has ``s = 0`` and codes 0;
* a block-scaled product sums over the K-blocks the dot product of the
  codes times both scales:
  ``h[r, n] = sum_kb sx[r, kb] * sw[n // 128, kb] * sum_{k in kb} qx[r, k] * qw[n, k]``
  (float64 here; the hardware accumulates in float32);
* the SwiGLU output is rounded to bfloat16 (as in the BF16 path) and then
  quantized per 1 x 128 block, like the dispatch rows, before the down
  projection; the router weight multiplies the down projection's result.
"""

import numpy as np

from .numerics import bf16_bits_to_f32, f32_to_bf16_bits, e4m3fn_round, E4M3FN_MAX
from .quant import quantize_weight_blocks
from .ffn import silu


def quantize_rows_fp8(x_bits, block: int = 128, row_mask=None):
    """The dispatch quantizer's output: E4M3 codes (as exact float64 values)
    and float32 scales per 1 x ``block`` block of bfloat16 rows [R, H].

    Returns ``(q float64 [R, H], s float32 [R, H/block])``.  Rows where
    ``row_mask`` is False (padding) get codes 0 and scales 0.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, H = x_bits.shape
    if H % block:
        raise ValueError("H must be a multiple of the block size")
    x = bf16_bits_to_f32(x_bits).reshape(R, H // block, block)
    amax = np.abs(x).max(axis=2)                                   # exact
    s = (amax / np.float32(E4M3FN_MAX)).astype(np.float32)         # IEEE division
    sb = s[:, :, None]
    safe = np.where(sb > 0, sb, np.float32(1))
    with np.errstate(over="ignore"):
        r = (x / safe).astype(np.float32)                          # IEEE division
    r = np.clip(r, -E4M3FN_MAX, E4M3FN_MAX)
    q = np.where(sb > 0, e4m3fn_round(r), 0.0).reshape(R, H)
    if row_mask is not None:
        keep = ~np.asarray(row_mask, dtype=bool)
        q[keep] = 0.0
        s = s.copy()
        s[keep] = 0
    return q, s


def block_scaled_matmul(qa, sa, qb, sb, block: int = 128):
    """``out[m, n] = sum_kb sa[m, kb] * sb[n // block, kb] * (qa[m, kb-block] . qb[n, kb-block])``.

    ``qa`` [M, K], ``sa`` [M, K/block] (per-row blocks), ``qb`` [N, K],
    ``sb`` [N/block, K/block] (tiles).  float64 throughout."""
    qa = np.asarray(qa, dtype=np.float64)
    qb = np.asarray(qb, dtype=np.float64)
    M, K = qa.shape
    N = qb.shape[0]
    out = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // block):
        ks = slice(kb * block, (kb + 1) * block)
        part = qa[:, ks] @ qb[:, ks].T                             # [M, N]
        row = np.asarray(sa, dtype=np.float64)[:, kb][:, None]
        col = np.repeat(np.asarray(sb, dtype=np.float64)[:, kb], block)[None, :N]
        out += part * row * col
    return out


def expert_ffn_w8a8_steps(qx, sx, w13_bits, w2_bits):
    """One expert's FFN on FP8 rows ``(qx, sx)`` [n, H] with the bfloat16
    weights quantized to 128 x 128 tiles, step by step: gate/up block-scaled
    product, ``a = bf16(silu(g) * u)``, ``a`` quantized per 1 x 128 block
    into ``(qa, sa)``, down block-scaled product ``y`` (float64 [n, H],
    before the router weight).  Returns ``{"qa", "sa", "y", "w2q"}`` where
    ``w2q = (q2, s2)`` is the down projection's quantized weight, so that a
    caller can also run the down product on other intermediate codes."""
    q13, s13, _ = quantize_weight_blocks(w13_bits)
    q2, s2, _ = quantize_weight_blocks(w2_bits)
    h = block_scaled_matmul(qx, sx, q13, s13)
    inter = q13.shape[0] // 2
    a = silu(h[:, :inter]) * h[:, inter:]
    a_bits = f32_to_bf16_bits(a.astype(np.float32))
    qa, sa = quantize_rows_fp8(a_bits)
    return {"qa": qa, "sa": sa, "y": block_scaled_matmul(qa, sa, q2, s2), "w2q": (q2, s2)}


def expert_ffn_w8a8(qx, sx, w13_bits, w2_bits):
    """``expert_ffn_w8a8_steps(...)["y"]``: float64 [n, H] before the router
    weight."""
    return expert_ffn_w8a8_steps(qx, sx, w13_bits, w2_bits)["y"]


def grouped_ffn_w8a8(qx, sx, cu_seqlens, counts, weights, row_scale=None):
    """Segment loop over expert-contiguous FP8 rows (``qx`` [cap, H] code
    values, ``sx`` [cap, H/128] scales); ``weights(e)`` gives expert e's
    bfloat16 ``(w13, w2)`` bits.  Rows past ``counts`` are not computed (0).
    Returns float64 [cap, H]."""
    cap, H = np.asarray(qx).shape
    y = np.zeros((cap, H), dtype=np.float64)
    for e in range(len(counts)):
        n = int(counts[e])
        if n == 0:
            continue
        r0 = int(cu_seqlens[e])
        w13, w2 = weights(e)
        ye = expert_ffn_w8a8(qx[r0:r0 + n], sx[r0:r0 + n], w13, w2)
        if row_scale is not None:
            ye = ye * np.asarray(row_scale[r0:r0 + n], dtype=np.float64)[:, None]
        y[r0:r0 + n] = ye
    return y
