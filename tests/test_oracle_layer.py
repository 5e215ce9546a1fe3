"""The oracle layer composed end to end on the tiny workload, and the input
recipe's properties (segment-size ranges, padding share, hot experts)."""

import numpy as np
import pytest

import oracle
import workloads
from oracle.numerics import bf16_bits_to_f64


def _tiny_layer(cfg, **kw):
    w = {e: workloads.expert_weights(cfg, e) for e in range(cfg.E)}
    return oracle.moe_layer(workloads.logits(cfg), workloads.hidden(cfg), lambda e: w[e],
                            cfg.K, workloads.row_valid(cfg), **kw), w


def test_layer_equals_dense_per_token_sum():
    """The grouped path equals a dense per-token loop over each token's
    experts (the MoonEP page's dense per-token reference MoE)."""
    cfg = workloads.CONFIGS["tiny"]
    res, w = _tiny_layer(cfg)
    x = bf16_bits_to_f64(workloads.hidden(cfg))
    for t in range(cfg.T):
        dense = np.zeros(cfg.H)
        for k in range(cfg.K):
            e = res["topk_idx"][t, k]
            dense += float(res["topk_w"][t, k]) * oracle.expert_ffn(x[t:t + 1], *w[e])[0]
        got = bf16_bits_to_f64(res["out"][t])
        # out is the sum of K bf16-rounded rows, rounded once more
        assert np.linalg.norm(got - dense) <= 1e-2 * np.linalg.norm(dense)


def test_layer_padding_rows_are_zero_and_shared_is_added():
    cfg = workloads.CONFIGS["tiny"].with_(pad_rows=7, shared_I=128)
    res, _ = _tiny_layer(cfg, shared_weights=workloads.shared_weights(cfg))
    pad = workloads.row_valid(cfg) == 0
    assert pad.sum() == 7
    # a padding token gets only the shared expert's row
    np.testing.assert_array_equal(res["out"][pad], res["shared"][pad])
    res2, _ = _tiny_layer(cfg)
    assert np.all(res2["out"][pad] == 0)


def test_layer_quant_options_change_output_within_fp8_error():
    cfg = workloads.CONFIGS["tiny"]
    base, _ = _tiny_layer(cfg)
    dq, _ = _tiny_layer(cfg, dispatch_block=128, pad_pow2=True)
    cq, _ = _tiny_layer(cfg, combine_qdq=True)
    ref = bf16_bits_to_f64(base["out"])
    for r in (dq, cq):
        d = bf16_bits_to_f64(r["out"])
        rel = np.linalg.norm(d - ref) / np.linalg.norm(ref)
        assert 1e-3 < rel < 0.1
    # calibration saw exactly the routed rows
    routed = cq["perm"]["src_of"] >= 0
    assert cq["combine_scale"] == np.float32(np.abs(bf16_bits_to_f64(cq["rows"][routed])).max().astype(np.float32) / np.float32(448))


def test_workload_shapes_and_recipe():
    c = workloads.CONFIGS
    assert (c["balanced"].T, c["balanced"].H, c["balanced"].E, c["balanced"].K, c["balanced"].I) == (512, 2048, 64, 8, 1024)
    assert c["prefill"].pad_rows == int(0.1 * 16384)
    lg = workloads.logits(c["balanced"])
    idx, _ = oracle.route(lg, None, 8)
    counts = np.bincount(idx.reshape(-1), minlength=64)
    assert 30 <= counts.min() and counts.max() <= 100
    lg2 = workloads.logits(c["skewed"])
    idx2, _ = oracle.route(lg2, None, 8)
    counts2 = np.bincount(idx2.reshape(-1), minlength=64)
    hot = workloads.hot_experts(c["skewed"])
    cold = np.setdiff1d(np.arange(64), hot)
    assert counts2[hot].min() > 4 * counts2[cold].max()
    v = workloads.row_valid(c["prefill"])
    assert int((v == 0).sum()) == 1638
