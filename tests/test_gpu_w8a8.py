"""The FP8 matrix-core path: FP8 rows, FP8 weights, block scales per K-block.

* moe_quant_rows_fp8 against oracle.quantize_rows_fp8: codes (decoded from
  their E4M3 bit fields, sign of zero included) and scales bit-exact, padding
  rows skipped, scales in the documented K-block-major layout.
* moe_pack_ffn_weights_fp8 with the K=128 layout: codes and scales
  bit-exact against oracle.quantize_weight_blocks through the documented
  order.
* moe_grouped_ffn_w8a8 against the oracle's FP8 FFN (float64, the same
  quantization of rows, weights and intermediate), in two steps, because one
  intermediate code that lands on the neighbouring E4M3 value (when the GPU's
  float32 SwiGLU and the oracle's float64 one round ``a`` to different bf16
  neighbours) moves its whole output row by up to ~2 % at I = 128: the
  intermediate codes and scales the gate/up stage leaves in the workspace
  equal the oracle's except for such rare neighbouring-code flips; the down
  stage, given the GPU's own intermediate, matches the oracle per row and
  element within 2e-2; and end to end the Frobenius error per expert is
  within 2e-2.  pow2 padding rows are never written; GATE_UP then DOWN gives
  the same bits as ALL.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_top_route_moe_amd import ops
from oracle.numerics import bf16_bits_to_f32
from tests.gpu_util import (need_gpu, dev_bf16, host_bits, dev, host, stacked_weights, check_rows,
                            rel_err, e4m3_decode, w8a8_intermediate, check_fp8_intermediate)

pytestmark = pytest.mark.gpu

FFN_TOL = 2e-2


def setup_module(module):
    need_gpu()
    assert ops.moe_device_check(0) == 0, "not a gfx950 device"


def test_quant_rows_fp8_matches_oracle():
    rng = np.random.default_rng(5)
    R, H = 77, 384
    x = (rng.standard_normal((R, H)) * np.exp2(rng.integers(-8, 8, (R, 1)))).astype(np.float32)
    x[3, 128:256] = 0.0                     # an all-zero block
    x[4, :] = -0.0                          # negative zeros
    x[5, 7] = 3e-38                         # far below the block's E4M3 range
    xb = oracle.f32_to_bf16_bits(x)
    src = np.arange(R, dtype=np.int32)
    src[[10, 40, 76]] = -1                  # padding rows
    stride = R + 13
    codes, scales = ops.moe_quant_rows_fp8(dev_bf16(xb), dev(src),
                                           scales=torch.full((H // 128, stride), 7.0, device="cuda"))
    torch.cuda.synchronize()
    q_want, s_want = oracle.quantize_rows_fp8(xb, row_mask=src >= 0)
    got_s = host(scales)
    np.testing.assert_array_equal(got_s[:, :R].T.view(np.uint32), s_want.view(np.uint32))
    assert np.all(got_s[:, R:] == 7.0)      # nothing past n_rows is written
    vals = e4m3_decode(host(codes))
    np.testing.assert_array_equal(vals, q_want)
    np.testing.assert_array_equal(np.signbit(vals), np.signbit(q_want))


@pytest.mark.parametrize("arrange", ["shuffled", "sorted"])
def test_quant_rows_fp8_exhaustive(arrange):
    """Every finite bfloat16 value once, in 1 x 128 blocks of mixed magnitude
    (shuffled) or of similar magnitude (sorted: every scale range, including
    the subnormal and the largest blocks, whose scales lie outside the
    reciprocal's exact range, where the kernel divides): codes, their signs
    and the scales bit-exact with the oracle."""
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(bf16_bits_to_f32(bits))]
    if arrange == "shuffled":
        bits = np.random.default_rng(13).permutation(bits)
    else:
        bits = bits[np.argsort(np.abs(bf16_bits_to_f32(bits)), kind="stable")]
    H = 512
    bits = np.concatenate([bits, np.zeros((-len(bits)) % H, np.uint16)]).reshape(-1, H)
    R = bits.shape[0]
    codes, scales = ops.moe_quant_rows_fp8(dev_bf16(bits))
    torch.cuda.synchronize()
    q_want, s_want = oracle.quantize_rows_fp8(bits)
    s_got = host(scales)[:, :R].T
    if arrange == "sorted":                 # both fallback ranges are reached
        assert s_got[s_got > 0].min() < 2.0 ** -90 and s_got.max() > 2.0 ** 90
    np.testing.assert_array_equal(s_got.view(np.uint32), s_want.view(np.uint32))
    vals = e4m3_decode(host(codes))
    np.testing.assert_array_equal(vals, q_want)
    np.testing.assert_array_equal(np.signbit(vals), np.signbit(q_want))


def unpack_k128(q: np.ndarray, gate_up: bool, G: int, N: int, Kdim: int) -> np.ndarray:
    """K=128-layout codes back to row-major [G, N, Kdim]: 16-byte unit
    ((((g * Kdim/128 + kb) * n_ct + ct) * 4 + f) * 2 + h) * 64 + l holds row
    row0(ct, f) + l % 16, columns 128 kb + 64 h + 16 (l / 16) .. +16."""
    def order(p):          # g kb ct f h l4 l16 c -> g ct f l16 kb h l4 c
        return p.transpose(0, 2, 3, 6, 1, 4, 5, 7)
    if not gate_up:
        p = q.reshape(G, Kdim // 128, N // 64, 4, 2, 4, 16, 16)
        return order(p).reshape(G, N, Kdim)
    I = N // 2
    p = q.reshape(G, Kdim // 128, I // 32, 4, 2, 4, 16, 16)
    gate = order(p[:, :, :, :2]).reshape(G, I, Kdim)
    up = order(p[:, :, :, 2:]).reshape(G, I, Kdim)
    return np.concatenate([gate, up], axis=1)


def test_pack_k128_layout_matches_oracle():
    G, H, I = 2, 384, 256
    cfg = workloads.MoEConfig("t", 23, T=8, H=H, E=G, K=1, I=I)
    w13, w2, host_w = stacked_weights(cfg)
    w13q, w13s, w2q, w2s = ops.moe_pack_ffn_weights_fp8(w13, w2, k128=True)
    torch.cuda.synchronize()
    for q, s, gate_up, N, Kd, idx in ((w13q, w13s, True, 2 * I, H, 0), (w2q, w2s, False, H, I, 1)):
        codes = unpack_k128(host(q), gate_up, G, N, Kd)
        for g in range(G):
            want_q, want_s, _ = oracle.quantize_weight_blocks(host_w[g][idx])
            np.testing.assert_array_equal(host(s)[g].view(np.uint32), want_s.view(np.uint32))
            vals = e4m3_decode(codes[g])
            np.testing.assert_array_equal(vals, want_q)
            np.testing.assert_array_equal(np.signbit(vals), np.signbit(want_q))


@pytest.mark.parametrize("H,I,T,hot,pow2", [
    (256, 128, 40, 0, False),      # short segments (one live row half)
    (384, 256, 300, 2, True),      # partial column block in the down GEMM, pow2 padding
    (256, 256, 2000, 2, False),    # several m-tiles per expert
    (512, 384, 500, 0, False),     # an odd number of K-blocks in the down GEMM
])
def test_w8a8_ffn_matches_oracle(H, I, T, hot, pow2):
    G = 6
    cfg = workloads.MoEConfig("t", 24, T=T, H=H, E=G, K=2, I=I, hot_experts=hot)
    idx, w = oracle.route(workloads.logits(cfg), None, 2)
    hid = workloads.hidden(cfg)
    w13, w2, host_w = stacked_weights(cfg)
    w13q, w13s, w2q, w2s = ops.moe_pack_ffn_weights_fp8(w13, w2, k128=True)
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), G, 0, pow2)
    cap = p.x_perm.shape[0]
    xq, xs = ops.moe_quant_rows_fp8(p.x_perm, p.src_of)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.zeros(cap, H, dtype=torch.bfloat16, device="cuda")
    ops.moe_grouped_ffn_w8a8(xq, xs, p.cu_seqlens, p.counts, w13q, w13s, w2q, w2s, p.w_perm, y,
                             dev_error=err)
    ws = torch.empty(ops.moe_grouped_ffn_w8a8_workspace_bytes(cap, G, H, I), dtype=torch.uint8,
                     device="cuda")
    y2 = torch.zeros_like(y)
    ops.moe_grouped_ffn_w8a8(xq, xs, p.cu_seqlens, p.counts, w13q, w13s, w2q, w2s, p.w_perm, y2,
                             ops.MOE_FFN_GATE_UP, ws)
    ops.moe_grouped_ffn_w8a8(xq, xs, p.cu_seqlens, p.counts, w13q, w13s, w2q, w2s, p.w_perm, y2,
                             ops.MOE_FFN_DOWN, ws)
    torch.cuda.synchronize()
    assert host(err)[0] == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    ref = oracle.permute(idx, w, hid, G, 0, pow2)
    qx, sx = oracle.quantize_rows_fp8(ref["x_perm"], row_mask=ref["src_of"] >= 0)
    got = bf16_bits_to_f32(host_bits(y))
    # the intermediate the gate/up stage left in the workspace, per row
    qa_gpu, sa_gpu = w8a8_intermediate(ws, cap, G, I, ref["counts"], ref["cu_seqlens"])
    worst, flips = 0.0, 0.0
    for e in range(G):
        n, r0 = int(ref["counts"][e]), int(ref["cu_seqlens"][e])
        if n == 0:
            continue
        st = oracle.expert_ffn_w8a8_steps(qx[r0:r0 + n], sx[r0:r0 + n], *host_w[e])
        rs = ref["w_perm"][r0:r0 + n, None].astype(np.float64)
        # gate/up: the same codes and scales but for last-bit flips of bf16 a
        flips = max(flips, check_fp8_intermediate(qa_gpu[r0:r0 + n], sa_gpu[r0:r0 + n],
                                                  st["qa"], st["sa"], what=f"expert {e}"))
        # down, on the GPU's own intermediate: per row and element
        y_own = oracle.block_scaled_matmul(qa_gpu[r0:r0 + n], sa_gpu[r0:r0 + n], *st["w2q"]) * rs
        c = check_rows(got[r0:r0 + n], y_own, FFN_TOL, what=f"expert {e} ({n} rows), down")
        worst = max(worst, c["worst_row"])
        # end to end against the oracle's own chain
        assert rel_err(got[r0:r0 + n], st["y"] * rs) <= FFN_TOL, e
        seg_end = int(ref["cu_seqlens"][e + 1])
        if seg_end > r0 + n:
            assert np.all(host_bits(y[r0 + n:seg_end]) == 0)
    print(f"H={H} I={I} T={T}: worst down row rel err {worst:.3e}, intermediate code flips {flips:.2e}")


@pytest.mark.parametrize("bad", ["negative", "past_the_end"])
def test_w8a8_scale_gather_out_of_range_fails_closed(bad):
    """The FP8 path's gate/up gathers each row's activation scales through
    scale_src[r] // scale_div (the permute's src_of and K): an entry that is
    negative, or whose column lies past the scale array's stride, raises
    ROW_RANGE instead of reading outside the array; the correct map raises
    nothing."""
    G, H, I, T, K = 2, 256, 256, 50, 2
    cfg = workloads.MoEConfig("t", 46, T=T, H=H, E=G, K=K, I=I)
    w13, w2, _ = stacked_weights(cfg)
    w13q, w13s, w2q, w2s = ops.moe_pack_ffn_weights_fp8(w13, w2, k128=True)
    xq_tok, xs = ops.moe_quant_rows_fp8(dev_bf16(workloads.hidden(cfg)))   # [T, H], [H/128, T]
    cap = T * K
    xq = xq_tok.repeat_interleave(K, dim=0).contiguous()   # row r holds token r // K
    counts, cu = np.array([60, 40], np.int32), np.array([0, 60, cap], np.int32)
    src = np.arange(cap, dtype=np.int32)

    def run(src_map):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        y = torch.zeros(cap, H, dtype=torch.bfloat16, device="cuda")
        ops.moe_grouped_ffn_w8a8(xq, xs, dev(cu), dev(counts), w13q, w13s, w2q, w2s, None, y,
                                 dev_error=err, scale_src=dev(src_map), scale_div=K)
        torch.cuda.synchronize()
        return int(host(err)[0])

    assert run(src) == 0
    corrupt = src.copy()
    if bad == "negative":
        corrupt[5] = -1
    else:
        corrupt[70] = T * K        # column T: one past the last token's
    assert run(corrupt) == ops.MOE_DEVERR_ROW_RANGE
