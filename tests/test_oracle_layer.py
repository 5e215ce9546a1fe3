"""The oracle layer composed end to end on the tiny workload, and the input
recipe's properties (segment-size ranges, padding share, hot experts)."""

import numpy as np

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


def _f32_ordered_sum(rows, shared=None):
    """float32 sum from +0 in the given order, the shared row last, then one
    bfloat16 rounding (written out here with scalar float32 adds)."""
    H = rows.shape[1] if len(rows) else shared.shape[0]
    acc = np.zeros(H, np.float32)
    for r in rows:
        acc = (acc + oracle.bf16_bits_to_f32(r)).astype(np.float32)
    if shared is not None:
        acc = (acc + oracle.bf16_bits_to_f32(shared)).astype(np.float32)
    return oracle.f32_to_bf16_bits(acc)


def test_layer_fp8_gemm_equals_dense_per_token_sum():
    """The FP8 path (``fp8_gemm=True``) through the grouped layer equals a
    dense per-token loop: quantize the token's row, run each chosen expert's
    FP8 FFN on that one row, weight it, round it to bfloat16, add the slots
    in order and the shared expert (on the same codes) last.  Pins the
    gather of codes and scales through ``src_of // K`` and the shared
    expert's input in the layer's FP8 branch."""
    cfg = workloads.CONFIGS["tiny"].with_(pad_rows=6, shared_I=128, T=24)
    sw = workloads.shared_weights(cfg)
    res, w = _tiny_layer(cfg, shared_weights=sw, fp8_gemm=True, pad_pow2=True)
    hid = workloads.hidden(cfg)
    for t in range(cfg.T):
        qx, sx = oracle.quantize_rows_fp8(hid[t:t + 1])
        rows = []
        for k in range(cfg.K):
            e = res["topk_idx"][t, k]
            if e < 0:
                continue
            y = oracle.expert_ffn_w8a8(qx, sx, *w[e])[0] * float(res["topk_w"][t, k])
            rows.append(oracle.f32_to_bf16_bits(y.astype(np.float32)))
        rows = np.array(rows, np.uint16).reshape(-1, cfg.H)
        shared = oracle.f32_to_bf16_bits(oracle.expert_ffn_w8a8(qx, sx, *sw)[0].astype(np.float32))
        np.testing.assert_array_equal(res["out"][t], _f32_ordered_sum(rows, shared), err_msg=str(t))


def test_layer_quantizer_wiring_equals_per_token_composition():
    """Dispatch and combine FP8 quantizers in the layer, bit for bit against
    a per-token composition: the token's row fake-quantized per 1 x 128
    block -> each chosen expert's FFN -> router weight -> bfloat16 -> the
    per-tensor combine QDQ -> the ordered sum, with the shared expert on the
    unquantized row, added last and never quantized.  The calibrated scale
    is fl32(max|row| / 448) over exactly the routed rows of the composition
    (pow2 padding rows and the shared rows excluded)."""
    cfg = workloads.CONFIGS["tiny"].with_(pad_rows=5, shared_I=128)
    sw = workloads.shared_weights(cfg)
    res, w = _tiny_layer(cfg, shared_weights=sw, dispatch_block=128, pad_pow2=True,
                         combine_qdq=True)
    hid = workloads.hidden(cfg)
    per_tok = []
    for t in range(cfg.T):
        if res["topk_idx"][t, 0] < 0:
            per_tok.append(np.zeros((0, cfg.H), np.uint16))
            continue
        hq, _ = oracle.fake_quant_block(hid[t:t + 1], 128)
        x = bf16_bits_to_f64(hq)
        rows = [oracle.f32_to_bf16_bits(
                    (oracle.expert_ffn(x, *w[res["topk_idx"][t, k]])[0]
                     * float(res["topk_w"][t, k])).astype(np.float32))
                for k in range(cfg.K)]
        per_tok.append(np.array(rows, np.uint16))
    allrows = np.concatenate([r for r in per_tok if len(r)])
    amax = np.float32(np.abs(oracle.bf16_bits_to_f32(allrows)).max())
    scale = np.float32(amax / np.float32(448.0))
    assert res["combine_scale"] == scale
    x_all = bf16_bits_to_f64(hid)
    for t in range(cfg.T):
        rows_q = oracle.fake_quant_per_tensor(per_tok[t], scale) if len(per_tok[t]) else per_tok[t]
        shared = oracle.f32_to_bf16_bits(oracle.expert_ffn(x_all[t:t + 1], *sw)[0].astype(np.float32))
        np.testing.assert_array_equal(res["out"][t], _f32_ordered_sum(rows_q, shared), err_msg=str(t))
