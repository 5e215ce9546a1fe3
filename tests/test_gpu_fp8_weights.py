"""FP8 expert weights (E4M3 codes with one float32 scale per 128 x 128 tile).

* moe_pack_ffn_weights_fp8 against oracle.quantize_weight_blocks: scales and
  codes bit-exact (codes read back through the packed order the header
  documents and decoded from the E4M3 bit fields, sign of zero included).
* moe_grouped_ffn_fp8 against moe_grouped_ffn run on the oracle's
  dequantized bf16 weights: bit-exact (the FP8 path dequantizes each weight
  to exactly that bf16 value before the same matrix-core sums), and against
  the float64 oracle FFN on those weights within the FFN tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_top_route_moe_amd import ops
from oracle.numerics import bf16_bits_to_f32
from tests.gpu_util import need_gpu, dev_bf16, host_bits, dev, host, stacked_weights, check_rows

pytestmark = pytest.mark.gpu

FFN_TOL = 2e-2


def setup_module(module):
    need_gpu()
    assert ops.moe_device_check(0) == 0, "not a gfx950 device"


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN bytes to values: sign bit, 4 exponent bits (bias 7), 3
    mantissa bits; exponent 0 is subnormal (m/8 * 2^-6).  The NaN codes
    (S.1111.111) must not appear."""
    c = codes.astype(np.int64)
    assert not np.any((c & 0x7F) == 0x7F), "NaN code"
    e, m = (c >> 3) & 0xF, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.where(c & 0x80, -mag, mag)


def unpack_codes(q: np.ndarray, gate_up: bool, G: int, N: int, Kdim: int) -> np.ndarray:
    """Packed codes back to row-major [G, N, Kdim]: 8-byte unit
    ((g * Kdim/32 + ks) * n_ct + ct) * 256 + f * 64 + l holds row
    row0(ct, f) + l % 16, columns 32 ks + 8 (l / 16) .. +8."""
    if not gate_up:
        p = q.reshape(G, Kdim // 32, N // 64, 4, 4, 16, 8)        # g ks ct f l4 l16 j
        return p.transpose(0, 2, 3, 5, 1, 4, 6).reshape(G, N, Kdim)
    I = N // 2
    p = q.reshape(G, Kdim // 32, I // 32, 4, 4, 16, 8)
    gate = p[:, :, :, :2].transpose(0, 2, 3, 5, 1, 4, 6).reshape(G, I, Kdim)
    up = p[:, :, :, 2:].transpose(0, 2, 3, 5, 1, 4, 6).reshape(G, I, Kdim)
    return np.concatenate([gate, up], axis=1)


def _plant_special_tiles(w13h, w2h):
    """Edge tiles: all zero (scale 0), one large value over tiny ones (E4M3
    subnormal codes and codes that round to zero), negative zeros."""
    w13h = w13h.copy()
    w2h = w2h.copy()
    w13h[0, 0:128, 0:128] = 0
    t = w13h[0, 128:256, 128:256]
    t[:] = (t & 0x8000) | 0x3000                       # +-2^-31
    t[5, 7] = 0x4300                                   # 128
    t[6, 9] = 0x8000                                   # -0
    w2h[-1, -128:, -128:] = 0x8000                     # a tile of -0 (amax 0)
    return w13h, w2h


@pytest.mark.parametrize("H,I,G", [(256, 128, 3), (384, 256, 2)])
def test_pack_fp8_weights_match_oracle(H, I, G):
    cfg = workloads.MoEConfig("t", 21, T=8, H=H, E=G, K=1, I=I)
    _, _, host_w = stacked_weights(cfg)
    w13h = np.stack([host_w[e][0] for e in range(G)])
    w2h = np.stack([host_w[e][1] for e in range(G)])
    w13h, w2h = _plant_special_tiles(w13h, w2h)
    w13q, w13s, w2q, w2s = ops.moe_pack_ffn_weights_fp8(dev_bf16(w13h), dev_bf16(w2h))
    torch.cuda.synchronize()
    for wh, q, s, gate_up, N, Kd in ((w13h, w13q, w13s, True, 2 * I, H),
                                     (w2h, w2q, w2s, False, H, I)):
        got_codes = unpack_codes(host(q), gate_up, G, N, Kd)
        got_s = host(s)
        for g in range(G):
            want_q, want_s, _ = oracle.quantize_weight_blocks(wh[g])
            np.testing.assert_array_equal(got_s[g].view(np.uint32), want_s.view(np.uint32))
            vals = e4m3_decode(got_codes[g])
            np.testing.assert_array_equal(vals, want_q)
            np.testing.assert_array_equal(np.signbit(vals), np.signbit(want_q))
    assert host(w13s)[0, 0, 0] == 0
    assert np.all(unpack_codes(host(w13q), True, G, 2 * I, H)[0, :128, :128] == 0)


def _dequantized(wh):
    return np.stack([oracle.quantize_weight_blocks(wh[g])[2] for g in range(wh.shape[0])])


@pytest.mark.parametrize("H,I,T,hot,pow2", [
    (256, 128, 40, 0, False),      # short segments: 4-wave workgroups
    (384, 256, 300, 2, True),      # partial column block, pow2 padding
    (256, 256, 2000, 2, False),    # long segments: 8-wave gate/up, several m-tiles
    (512, 256, 500, 0, False),     # mean of 1-2 m-tiles: 8-wave down projection
])
def test_ffn_fp8_weights_equal_bf16_on_dequantized(H, I, T, hot, pow2):
    G = 6
    cfg = workloads.MoEConfig("t", 22, T=T, H=H, E=G, K=2, I=I, hot_experts=hot)
    idx, w = oracle.route(workloads.logits(cfg), None, 2)
    hid = workloads.hidden(cfg)
    _, _, host_w = stacked_weights(cfg)
    w13h = np.stack([host_w[e][0] for e in range(G)])
    w2h = np.stack([host_w[e][1] for e in range(G)])
    w13h, w2h = _plant_special_tiles(w13h, w2h)
    w13q, w13s, w2q, w2s = ops.moe_pack_ffn_weights_fp8(dev_bf16(w13h), dev_bf16(w2h))
    d13, d2 = _dequantized(w13h), _dequantized(w2h)
    d13p, d2p = ops.moe_pack_ffn_weights(dev_bf16(d13), dev_bf16(d2))

    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), G, 0, pow2)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y8 = torch.zeros(p.x_perm.shape, dtype=torch.bfloat16, device="cuda")
    ops.moe_grouped_ffn_fp8(p.x_perm, p.cu_seqlens, p.counts, w13q, w13s, w2q, w2s, p.w_perm,
                            y8, dev_error=err)
    yb = torch.zeros_like(y8)
    ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, d13p, d2p, p.w_perm, yb,
                        flags=ops.MOE_FFN_ALL | ops.MOE_FFN_PACKED_WEIGHTS)
    assert host(err)[0] == 0
    # the same tiles (128-row, or the streamed 256-row tiles for segments
    # averaging 96..255 rows), the same summation order: the
    # same bits
    assert torch.equal(y8.view(torch.int16), yb.view(torch.int16))
    # the stages run separately give the same bits
    ws = torch.empty(ops.moe_grouped_ffn_workspace_bytes(p.x_perm.shape[0], G, H, I),
                     dtype=torch.uint8, device="cuda")
    y2 = torch.zeros_like(y8)
    ops.moe_grouped_ffn_fp8(p.x_perm, p.cu_seqlens, p.counts, w13q, w13s, w2q, w2s, p.w_perm,
                            y2, ops.MOE_FFN_GATE_UP, ws)
    ops.moe_grouped_ffn_fp8(p.x_perm, p.cu_seqlens, p.counts, w13q, w13s, w2q, w2s, p.w_perm,
                            y2, ops.MOE_FFN_DOWN, ws)
    assert torch.equal(y8.view(torch.int16), y2.view(torch.int16))
    # and the float64 oracle on the dequantized weights
    ref = oracle.permute(idx, w, hid, G, 0, pow2)
    for e in range(G):
        n, r0 = int(ref["counts"][e]), int(ref["cu_seqlens"][e])
        if n == 0:
            continue
        x = oracle.bf16_bits_to_f64(ref["x_perm"][r0:r0 + n])
        want = oracle.expert_ffn(x, d13[e], d2[e]) * ref["w_perm"][r0:r0 + n, None].astype(np.float64)
        check_rows(bf16_bits_to_f32(host_bits(y8[r0:r0 + n])), want, FFN_TOL, what=f"expert {e}")
        check_rows(bf16_bits_to_f32(host_bits(yb[r0:r0 + n])), want, FFN_TOL, what=f"bf16 expert {e}")
