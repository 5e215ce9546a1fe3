"""Oracle for routing: per-token top-k experts and their weights.

Test infrastructure only (see the package docstring).

Sources:
* "[Kernel] DeepEP dispatch-combine kernel integration", review threads on
  the prepare/finalize classes: the router hands the MoE layer per-token
  ``topk_ids`` / ``topk_weights`` of shape [T, K].
* "[Distributed][MoonEP] BF16 integration of MoonEP balanced EP backend",
  review thread on the MoonEP prepare/finalize: the layer consumes the
  original [T, K] routing ids.
* "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM Mega-MoE",
  review thread on the combine-buffer check: a slot is valid iff its
  ``topk_idx >= 0``; padding rows carry -1 in every slot.
* The workload descriptions fix the rule: softmax over the router logits,
  top-k, weights renormalised over the chosen k.

Readings where the pages are silent:
* slot 0 holds the largest logit, slots follow in descending logit order
  (the combine adds slots in increasing slot index, which presupposes some
  order of the slots);
* ties between equal logits go to the lower expert index;
* selection compares the float32 logits themselves (softmax is monotone, so
  this is the same ranking as by probability, and it is exact);
* with ``renormalize=False`` the weights are the full softmax over all E;
* non-finite logits: a NaN ranks as -inf (below every number); a logit
  equal to the row's largest chosen logit counts ``exp(0) = 1`` even when
  both are infinite (the limit of the softmax; for finite logits the same
  value), so a row whose chosen logits are all -inf gets ``1/k`` each.
"""

import numpy as np


def route(logits, row_valid=None, k: int = 1, renormalize: bool = True):
    """Return ``(topk_idx int32 [T,K], topk_w float32 [T,K])``.

    ``logits``: float32 [T, E].  ``row_valid``: optional bool/uint8 [T];
    rows with 0 are padding and get ``idx = -1`` and ``w = 0`` in every slot.
    Weights are ``exp(l_k - l_max) / sum_j exp(l_j - l_max)`` evaluated in
    float64 and stored as float32, the sum running over the selected k
    (renormalised) or over all E.
    """
    logits = np.asarray(logits, dtype=np.float32)
    logits = np.where(np.isnan(logits), np.float32(-np.inf), logits)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    idx = np.full((T, k), -1, dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float32)
    # descending by value; a stable sort keeps the lower index first among
    # equal values
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    l64 = logits.astype(np.float64)
    sel_l = np.take_along_axis(l64, order, axis=1)
    lmax = sel_l[:, :1]

    def term(l):
        with np.errstate(invalid="ignore"):
            return np.where(l == lmax, 1.0, np.exp(l - lmax))

    num = term(sel_l)
    if renormalize:
        den = num.sum(axis=1, keepdims=True)
    else:
        den = term(l64).sum(axis=1, keepdims=True)
    valid = np.ones(T, dtype=bool) if row_valid is None else np.asarray(row_valid).astype(bool)
    idx[valid] = order[valid]
    w[valid] = (num / den)[valid].astype(np.float32)
    return idx, w
