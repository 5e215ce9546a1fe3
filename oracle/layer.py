"""Oracle for the whole MoE layer, composed from the stage oracles.

Test infrastructure only (see the package docstring).

Order of the steps, as the pages put them together:
route ("[Kernel] DeepEP dispatch-combine kernel integration", review
threads: router ids and weights [T, K]) -> dispatch fake-quant of the expert
input tokens ("Add MoE dispatch/combine fake quantization for vLLM's
DeepGEMM Mega-MoE", "How it works") -> permute into expert segments
("[Distributed][MoonEP] BF16 integration of MoonEP balanced EP backend",
"Purpose") -> grouped SwiGLU FFN with the route weight applied before the
down projection (same page, commit message adding the modular experts) ->
BF16 per-(token, slot) rows, fake-quantized by the combine quantizer with a
calibrated or constant scale -> combine, lowest slot index first, with the
shared expert's unquantized slot last (first page, PR summary).

Readings where the pages are silent:
* the shared expert sees the layer input ``hidden`` (the first page keeps
  dispatch quantization and a fused shared expert apart, so no config has
  both) and its output is a BF16 row with weight 1, added for every token;
* combine-row quantization covers routed rows only; with no scale given it
  is calibrated from this batch's own rows (max calibration);
* FP8 expert weights (128 x 128 tile scales, the "DeepEP + DeepGEMM" review
  thread) enter the FFN as their dequantized values, for the routed and the
  shared experts alike;
* the real FP8 path (``fp8_gemm``) quantizes every row of the layer input
  per 1 x 128 block (the dispatch quantizer of the low-latency dispatch
  thread, handing over codes and scales), which replaces the dispatch
  fake-quant; routed and shared experts run the FP8 FFN of ``fp8_gemm.py``
  on those codes.
"""

import numpy as np

from .numerics import bf16_bits_to_f64, f32_to_bf16_bits
from .route import route
from .quant import (fake_quant_block, fake_quant_per_tensor, calibrate_amax, scale_from_amax,
                    quantize_weight_blocks)
from .fp4 import fake_quant_mxfp4, fake_quant_nvfp4, nvfp4_tensor_scale
from .permute import permute
from .ffn import grouped_ffn, expert_ffn
from .fp8_gemm import quantize_rows_fp8, grouped_ffn_w8a8, expert_ffn_w8a8
from .combine import combine


def _rows_to_bf16(y64):
    """float64 rows -> float32 (one rounding) -> bfloat16 bits.

    The float64 value is first rounded to binary32 and then to bfloat16;
    this double rounding only matters in the last bit of values that sit on
    a bfloat16 tie after the first rounding, well inside the FFN tolerance.
    """
    return f32_to_bf16_bits(np.asarray(y64, dtype=np.float64).astype(np.float32))


def moe_layer(logits, hidden_bits, weights, k: int, row_valid=None,
              renormalize: bool = True, dispatch_block=None, pad_pow2=False,
              shared_weights=None, combine_qdq: bool = False, combine_scale=None,
              expert_begin: int = 0, num_local_experts=None, dispatch_fp4=None,
              dispatch_scale=None, combine_fp4=None, fp8_weights: bool = False,
              fp8_gemm: bool = False):
    """Run the oracle layer and return every intermediate in a dict.

    ``weights(e)`` returns expert ``e``'s ``(w13, w2)`` as bfloat16 bits
    (global expert index).  ``shared_weights``: optional ``(w13, w2)``.
    ``dispatch_fp4`` / ``combine_fp4`` ("nvfp4" or "mxfp4") select the FP4
    quantizers instead of the FP8 ones; an NVFP4 tensor scale not given
    (``dispatch_scale``, ``combine_scale``) is calibrated like the FP8
    combine scale: ``amax / (6 * 448)`` over the rows the quantizer sees.
    ``fp8_weights``: every expert weight matrix is replaced by its FP8
    fake-quant with one scale per 128 x 128 tile.  ``fp8_gemm``: the real FP8
    path (rows and weights as codes with block scales; see the module
    readings).
    """
    if fp8_weights:
        def deq(w):
            return quantize_weight_blocks(w)[2]

        raw_weights = weights
        weights = lambda e: tuple(deq(w) for w in raw_weights(e))  # noqa: E731
        if shared_weights is not None:
            shared_weights = tuple(deq(w) for w in shared_weights)
    logits = np.asarray(logits, dtype=np.float32)
    hidden_bits = np.asarray(hidden_bits, dtype=np.uint16)
    T, E = logits.shape
    El = E if num_local_experts is None else num_local_experts

    topk_idx, topk_w = route(logits, row_valid, k, renormalize)
    valid_tok = (topk_idx >= 0).any(axis=1)

    dscale = None
    hq = hs = None
    if fp8_gemm:
        if dispatch_fp4:
            raise ValueError("the FP8 path has its own dispatch quantizer")
        hq, hs = quantize_rows_fp8(hidden_bits)
        hidden_q, dscales = hidden_bits, hs
    elif dispatch_fp4 == "mxfp4":
        hidden_q, dscales = fake_quant_mxfp4(hidden_bits, row_mask=valid_tok)
    elif dispatch_fp4 == "nvfp4":
        dscale = (nvfp4_tensor_scale(calibrate_amax(hidden_bits, valid_tok))
                  if dispatch_scale is None else np.float32(dispatch_scale))
        hidden_q, dscales = fake_quant_nvfp4(hidden_bits, dscale, row_mask=valid_tok)
    elif dispatch_block:
        hidden_q, dscales = fake_quant_block(hidden_bits, dispatch_block, row_mask=valid_tok)
    else:
        hidden_q, dscales = hidden_bits, None

    perm = permute(topk_idx, topk_w, hidden_q, El, expert_begin, pad_pow2, num_experts=E)
    if fp8_gemm:
        src = perm["src_of"]
        tok = np.where(src >= 0, src // k, 0)
        qx = np.where((src >= 0)[:, None], hq[tok], 0.0)
        sx = np.where((src >= 0)[:, None], hs[tok], np.float32(0))
        y = grouped_ffn_w8a8(qx, sx, perm["cu_seqlens"], perm["counts"],
                             lambda e: weights(e + expert_begin), row_scale=perm["w_perm"])
    else:
        y = grouped_ffn(perm["x_perm"], perm["cu_seqlens"], perm["counts"],
                        lambda e: weights(e + expert_begin), row_scale=perm["w_perm"])
    rows = _rows_to_bf16(y)
    routed_rows = perm["src_of"] >= 0

    scale = None
    rows_q = rows
    if combine_fp4 == "mxfp4":
        rows_q, _ = fake_quant_mxfp4(rows, row_mask=routed_rows)
    elif combine_fp4 == "nvfp4":
        scale = (nvfp4_tensor_scale(calibrate_amax(rows, routed_rows))
                 if combine_scale is None else np.float32(combine_scale))
        rows_q, _ = fake_quant_nvfp4(rows, scale, row_mask=routed_rows)
    elif combine_qdq:
        if combine_scale is None:
            scale = scale_from_amax(calibrate_amax(rows, routed_rows))
        else:
            scale = np.float32(combine_scale)
        rows_q = fake_quant_per_tensor(rows, scale, row_mask=routed_rows)

    shared = None
    if shared_weights is not None:
        s13, s2 = shared_weights
        if fp8_gemm:
            shared = _rows_to_bf16(expert_ffn_w8a8(hq, hs, s13, s2))
        else:
            shared = _rows_to_bf16(expert_ffn(bf16_bits_to_f64(hidden_bits), s13, s2))

    out = combine(rows_q, perm["row_of"], T, k, shared)
    return {
        "topk_idx": topk_idx, "topk_w": topk_w,
        "hidden_q": hidden_q, "dispatch_scales": dscales, "dispatch_scale": dscale,
        "perm": perm, "y": y, "rows": rows, "rows_q": rows_q,
        "combine_scale": scale, "shared": shared, "out": out,
    }
