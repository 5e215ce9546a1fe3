"""Oracle for the combine: the page's fixed summation order.

Test infrastructure only (see the package docstring).

Source: "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM
Mega-MoE", PR summary and "How it works": the per-(token, slot) rows are
re-added in the order the fused kernel uses — slot by slot with the lowest
valid slot index first, into a float32 sum that begins at zero, with a
single rounding to bf16 after the last add; a fused shared expert is added
after all routed slots and is never quantized.  A slot is valid iff its
``topk_idx >= 0`` (review thread on the buffer check).

Every add below is a numpy float32 elementwise add, i.e. one IEEE binary32
round-to-nearest-even operation, applied in exactly the page's order; there
is no fused multiply-add and no tree or pairwise reduction.
"""

import numpy as np

from .numerics import bf16_bits_to_f32, f32_to_bf16_bits


def combine(rows_bits, row_of, T: int, K: int, shared_bits=None):
    """``out[t] = bf16(((+0 + r_{t,k0}) + r_{t,k1}) + ... + shared[t])``.

    ``rows_bits``: uint16 [R, H] per-(token, slot) rows; ``row_of``: int32
    [T*K] with the row of slot ``(t, k)`` or a negative value for an invalid
    slot; ``shared_bits``: optional uint16 [T, H].  Returns uint16 [T, H].
    """
    rows_bits = np.asarray(rows_bits, dtype=np.uint16)
    row_of = np.asarray(row_of, dtype=np.int64).reshape(T, K)
    H = rows_bits.shape[1]
    acc = np.zeros((T, H), dtype=np.float32)             # +0.0
    for k in range(K):                                   # slot 0 first
        r = row_of[:, k]
        valid = r >= 0
        if not valid.any():
            continue
        add = bf16_bits_to_f32(rows_bits[r[valid]])
        acc[valid] = acc[valid] + add                    # binary32 add
    if shared_bits is not None:
        acc = acc + bf16_bits_to_f32(np.asarray(shared_bits, dtype=np.uint16))
    return f32_to_bf16_bits(acc)                         # the one rounding
