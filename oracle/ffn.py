"""Oracle for the expert SwiGLU FFN, per expert and over grouped segments.

Test infrastructure only (see the package docstring).

Sources:
* "[Distributed][MoonEP] BF16 integration of MoonEP balanced EP backend",
  commit message adding the modular experts: three grouped matmuls (gate,
  up, down) over the ``cu_seqlens`` segments, route weights applied before
  the down projection, empty segments skipped; the gate and up weights are
  the two halves of the layer's ``w13``; H and I multiples of 128.
* "[Kernel] DeepEP dispatch-combine kernel integration", review thread on
  the DeepEP + DeepGEMM test: ``w1`` has ``2n`` output rows (gate and up)
  and ``w2`` maps the ``n`` intermediate channels back to the hidden size.
* "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM Mega-MoE",
  "How it works": the kernel leaves router-weighted per-(token, slot) BF16
  rows.

Readings where the pages are silent:
* ``w13[e]`` is [2I, H] with gate rows [0, I) and up rows [I, 2I);
  ``w2[e]`` is [H, I] (both as ``y = x @ W.T``);
* the activation is SwiGLU, ``silu(g) * u`` with ``silu(z) = z / (1 + e^-z)``;
* the router weight multiplies the down projection's result (equal in
  exact arithmetic to weighting its input);
* all arithmetic here is float64 from the exact bfloat16 inputs: no
  intermediate rounding.  The per-(token, slot) rows are rounded to
  bfloat16 only where the pages say the rows are BF16 (the layer does that).
"""

import numpy as np

from .numerics import bf16_bits_to_f64


def silu(z):
    """``z * sigmoid(z)`` in float64, written to avoid exp overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def expert_ffn(x, w13, w2):
    """One expert's SwiGLU FFN on rows ``x`` (float64 [n, H]).

    ``w13``: [2I, H], ``w2``: [H, I] (float64 or bfloat16 bits).  Returns
    float64 [n, H] = ``(silu(x W_g^T) * (x W_u^T)) W_2^T``.
    """
    if np.asarray(w13).dtype == np.uint16:
        w13 = bf16_bits_to_f64(w13)
    if np.asarray(w2).dtype == np.uint16:
        w2 = bf16_bits_to_f64(w2)
    x = np.asarray(x, dtype=np.float64)
    inter = w13.shape[0] // 2
    g = x @ w13[:inter].T
    u = x @ w13[inter:].T
    a = silu(g) * u
    return a @ w2.T


def grouped_ffn(x_perm_bits, cu_seqlens, counts, weights, row_scale=None):
    """Segment loop over the expert-contiguous rows.

    ``x_perm_bits``: uint16 [cap, H]; segment e holds its ``counts[e]`` valid
    rows at ``cu_seqlens[e]``; rows past them (power-of-two padding) are not
    computed and come back as 0.  ``weights(e)`` returns expert e's
    ``(w13, w2)``.  ``row_scale``: optional float32 [cap] router weight per
    row.  Returns float64 [cap, H].
    """
    x_perm_bits = np.asarray(x_perm_bits, dtype=np.uint16)
    cap, H = x_perm_bits.shape
    y = np.zeros((cap, H), dtype=np.float64)
    for e in range(len(counts)):
        n = int(counts[e])
        if n == 0:
            continue                      # empty segments are skipped
        r0 = int(cu_seqlens[e])
        w13, w2 = weights(e)
        ye = expert_ffn(bf16_bits_to_f64(x_perm_bits[r0:r0 + n]), w13, w2)
        if row_scale is not None:
            ye = ye * np.asarray(row_scale[r0:r0 + n], dtype=np.float64)[:, None]
        y[r0:r0 + n] = ye
    return y
