"""Oracle for the permute: expert-contiguous segments of the routed rows.

Test infrastructure only (see the package docstring).

Sources:
* "[Distributed][MoonEP] BF16 integration of MoonEP balanced EP backend",
  "Purpose": the experts are handed rows that are already sorted by expert,
  an ``[NvS, H]`` matrix described by ``cu_seqlens`` with no per-token ids,
  so each expert works on one contiguous segment of it (a grouped GEMM).
* "[Bugfix][MoE] Size the permute scratch from its inputs", PR summary and
  "Details": the permute metadata is int32 arrays over the expanded rows,
  sized from the rows actually received (not predicted from a config), the
  permuted hidden states live in a caller buffer, and receive buckets may be
  rounded up to powers of two ("next_power_of_2").
* "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM Mega-MoE",
  review thread on the buffer check: a slot is routed iff ``topk_idx >= 0``.

Readings where the pages are silent:
* within a segment, rows are ordered by the flat slot index ``t*K + k``
  (a stable sort by expert), so every index array is unique;
* power-of-two mode rounds each expert's segment up to the next power of
  two (an empty segment stays empty); the valid rows come first and the
  padding rows after them carry ``src_of = -1`` and weight 0;
* an expert-parallel share is ``[expert_begin, expert_begin + E_local)``;
  slots routed elsewhere get ``row_of = -1``;
* a negative id is a padding slot (the buffer-check thread's validity
  test); an id at or past the layer's expert count names no expert, is not
  routed, and is reported (``expert_range_error``) — a corrupt router output
  fails closed (the same page's review thread on graph capture: a
  device-side check that records the failure).
"""

import numpy as np


def next_pow2(n: int) -> int:
    """Smallest power of two >= n, with 0 -> 0."""
    if n <= 0:
        return 0
    p = 1
    while p < n:
        p *= 2
    return p


def permute(topk_idx, topk_w, hidden_bits, num_local_experts: int,
            expert_begin: int = 0, pad_pow2: bool = False, num_experts=None):
    """Group the routed (token, slot) pairs by expert.

    ``num_experts`` (default: the end of the local range) is the layer's
    expert count; ``expert_range_error`` in the result says whether any id
    reached it.

    Returns a dict with ``counts [E_l]``, ``cu_seqlens [E_l+1]`` (int32),
    ``row_of [T*K]``, ``src_of [cap]`` (int32), ``w_perm [cap]`` (float32)
    and ``x_perm [cap, H]`` (uint16; padding rows are zero here and are never
    compared).  ``cap`` is ``cu_seqlens[-1]``.
    """
    topk_idx = np.asarray(topk_idx, dtype=np.int32)
    topk_w = np.asarray(topk_w, dtype=np.float32)
    hidden_bits = np.asarray(hidden_bits, dtype=np.uint16)
    T, K = topk_idx.shape
    H = hidden_bits.shape[1]
    El = num_local_experts

    if num_experts is None:
        num_experts = expert_begin + El
    flat = topk_idx.reshape(-1).astype(np.int64)
    local = flat - expert_begin
    routed = (flat >= 0) & (flat < num_experts) & (local >= 0) & (local < El)

    counts = np.bincount(local[routed], minlength=El).astype(np.int64)
    sizes = np.array([next_pow2(int(c)) for c in counts], dtype=np.int64) if pad_pow2 else counts
    cu = np.zeros(El + 1, dtype=np.int64)
    cu[1:] = np.cumsum(sizes)
    cap = int(cu[-1])

    row_of = np.full(T * K, -1, dtype=np.int32)
    src_of = np.full(cap, -1, dtype=np.int32)
    w_perm = np.zeros(cap, dtype=np.float32)
    x_perm = np.zeros((cap, H), dtype=np.uint16)
    fill = cu[:-1].copy()                          # next free row per expert
    for i in np.nonzero(routed)[0]:                # ascending flat index
        e = local[i]
        r = fill[e]
        fill[e] += 1
        row_of[i] = r
        src_of[r] = i
        w_perm[r] = topk_w.reshape(-1)[i]
        x_perm[r] = hidden_bits[i // K]
    return {
        "counts": counts.astype(np.int32),
        "cu_seqlens": cu.astype(np.int32),
        "row_of": row_of,
        "src_of": src_of,
        "w_perm": w_perm,
        "x_perm": x_perm,
        "expert_range_error": bool((flat >= num_experts).any()),
    }
