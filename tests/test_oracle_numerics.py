"""Pins of the oracle's number formats against independent implementations.

* bfloat16 rounding vs torch's CPU float32 -> bfloat16 cast (IEEE RNE).
* E4M3FN rounding vs torch's CPU float32 -> float8_e4m3fn cast (OCP RNE) on
  every bfloat16 value inside +-448 and on every tie point.
* the fake-quant composition vs the same steps done with torch ops.
* hand values from the format definitions.
"""

import numpy as np
import pytest
import torch
import oracle

from oracle.numerics import (
    bf16_bits_to_f32, f32_to_bf16_bits, e4m3fn_table, e4m3fn_round, qdq_e4m3fn,
)


def _torch_bf16_bits(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_on_random_bit_patterns():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    np.testing.assert_array_equal(f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_bf16_matches_torch_on_ties_and_edges():
    # every tie point of the bfloat16 grid around a range of binades
    base = np.arange(0, 2**16, dtype=np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    near = np.concatenate([(base | 0x7FFF), (base | 0x8001), base]).view(np.float32)
    x = np.concatenate([ties, near])
    x = x[~np.isnan(x)]
    np.testing.assert_array_equal(f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_bf16_hand_values():
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,          # tie -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 0x3F82,      # tie -> even (1 + 2^-6)
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,
        -0.0: 0x8000,
        2.0 ** -133: 0x0001,              # smallest bfloat16 subnormal
        float(np.finfo(np.float32).max): 0x7F80,   # overflows to +inf
    }
    for v, want in cases.items():
        assert int(f32_to_bf16_bits(np.float32(v))) == want, v
    assert int(f32_to_bf16_bits(np.float32(np.nan))) & 0x7FFF == 0x7FC0
    w = bf16_bits_to_f32(np.array([0x3F80, 0xC000, 0x0001], dtype=np.uint16))
    assert w[0] == 1.0 and w[1] == -2.0 and w[2] == np.float32(2.0 ** -133)


def test_e4m3fn_table_hand_values():
    t = e4m3fn_table()
    assert len(t) == 127
    assert np.all(np.diff(t) > 0)
    assert t[0] == 0.0
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0              # largest finite


def _torch_e4m3(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3fn_matches_torch_on_all_bf16_values_in_range():
    bits = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    x = bf16_bits_to_f32(bits)
    x = x[np.isfinite(x) & (np.abs(x) <= 448)]
    np.testing.assert_array_equal(e4m3fn_round(x), _torch_e4m3(x))


def test_e4m3fn_matches_torch_on_ties_and_random():
    t = e4m3fn_table()
    mids = ((t[1:] + t[:-1]) / 2).astype(np.float32)      # every tie point
    assert np.all(mids.astype(np.float64) == (t[1:] + t[:-1]) / 2)
    rng = np.random.default_rng(1)
    r = (rng.standard_normal(200_000) * rng.choice([1e-3, 0.1, 10, 100], 200_000)).astype(np.float32)
    r = np.clip(r, -448, 448)
    x = np.concatenate([mids, -mids, r])
    np.testing.assert_array_equal(e4m3fn_round(x), _torch_e4m3(x))


def test_e4m3fn_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3fn_round(np.array([449.0]))


def _torch_qdq(x_f32, s):
    x = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    s = torch.tensor(np.float32(s))
    q = torch.clamp(x / s, -448, 448).to(torch.float8_e4m3fn).to(torch.float32)
    return (q * s).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("s", [1.0, 2.0 ** -7, 0.0123, 3.7e-3, 1.0 / 448, 0.3])
def test_qdq_matches_torch_composition_exhaustively(s):
    bits = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    x = bf16_bits_to_f32(bits)
    x = x[np.isfinite(x)]
    np.testing.assert_array_equal(qdq_e4m3fn(x, np.float32(s)), _torch_qdq(x, s))


def test_qdq_invariants():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50_000) * 3).astype(np.float32)
    s = np.float32(np.abs(x).max() / np.float32(448))
    y = qdq_e4m3fn(x, s)
    yf = bf16_bits_to_f32(y)
    # idempotent: the outputs are (bf16 roundings of) grid points code * s
    np.testing.assert_array_equal(qdq_e4m3fn(yf, s), y)
    # the largest magnitude maps onto 448 * s
    i = np.argmax(np.abs(x))
    assert yf[i] == bf16_bits_to_f32(f32_to_bf16_bits(np.float32(448) * s * np.sign(x[i])))
    # error within half an e4m3 step (relative 2^-4 for normals) plus bf16
    big = np.abs(x / s) >= 2.0 ** -6
    rel = np.abs(yf[big] - x[big]) / np.abs(x[big])
    assert rel.max() <= 2.0 ** -4 + 2.0 ** -8
    # zero scale: all zero output
    assert np.all(qdq_e4m3fn(np.zeros(8, np.float32), np.float32(0)) == 0)


# ---------------------------------------------------------------- FP4 (E2M1)
# Hand-worked values; E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 and a
# tie goes to the code whose mantissa bit is 0.

def test_e2m1_grid_and_ties():
    from oracle.fp4 import e2m1_table
    np.testing.assert_array_equal(e2m1_table(), [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    cases = {0.0: 0, 0.2: 0, 0.25: 0, 0.3: 0.5, 0.5: 0.5, 0.75: 1, 1.0: 1, 1.25: 1, 1.3: 1.5,
             1.75: 2, 2.4: 2, 2.5: 2, 2.6: 3, 3.5: 4, 4.9: 4, 5.0: 4, 5.1: 6, 6.0: 6}
    for v, want in cases.items():
        assert oracle.e2m1_round(v) == want, v
        assert oracle.e2m1_round(-v) == -want, -v
    assert np.signbit(oracle.e2m1_round(-0.1))             # the sign survives a zero


def _bf(vals):
    return f32_to_bf16_bits(np.asarray(vals, np.float32))


def test_mxfp4_hand_examples():
    # block 0: amax 1 -> scale 2^(0-2) = 0.25; block 1: amax 7.875 -> scale 1,
    # 7.875 saturates to 6; block 2: amax 3.984375 -> floor(log2) = 1 -> scale
    # 0.5, 7.97 saturates to 6 -> 3; block 3: all zero
    b0 = [1.0, 0.3, -0.6, 0.1, 0.0625] + [0.0] * 27
    b1 = [7.875, -2.5, 0.75] + [0.0] * 29
    b2 = [3.984375, 1.25] + [0.0] * 30
    b3 = [0.0] * 32
    x = _bf([b0 + b1 + b2 + b3])
    out, X = oracle.fake_quant_mxfp4(x)
    np.testing.assert_array_equal(X, [[0.25, 1.0, 0.5, 0.0]])
    got = bf16_bits_to_f32(out)[0]
    # 0.3/0.25 = 1.2 -> 1; -0.6/0.25 = -2.4 -> -2; 0.1/0.25 -> 0.5 (bf16 0.1 is
    # 0.10009765625, 0.4004 -> 0.5); 0.0625/0.25 = 0.25 -> tie -> 0
    np.testing.assert_array_equal(got[:5], [1.0, 0.25, -0.5, 0.125, 0.0])
    np.testing.assert_array_equal(got[32:35], [6.0, -2.0, 1.0])     # -2.5 tie -> -2
    np.testing.assert_array_equal(got[64:66], [3.0, 1.0])           # 1.25/0.5 = 2.5 -> 2
    assert np.all(out[0, 96:] == 0)


def test_mxfp4_scale_exponent_clamp():
    # amax 2^-130 (a bfloat16 subnormal): floor(log2) - 2 = -132 clamps to
    # -127, so x / 2^-127 = 2^-3 rounds to +0
    tiny = np.uint16(0x0008)                                # 2^-130 in bfloat16
    assert bf16_bits_to_f32(np.array([tiny]))[0] == np.float32(2.0 ** -130)
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = tiny
    out, X = oracle.fake_quant_mxfp4(x)
    assert X[0, 0] == 2.0 ** -127 and np.all(out == 0)
    # a huge block: amax 2^127 -> scale 2^125; 2^127 / 2^125 = 4 exactly
    x[0, 0] = np.uint16(0x7F00)                             # 2^127
    out, X = oracle.fake_quant_mxfp4(x)
    assert X[0, 0] == 2.0 ** 125 and out[0, 0] == np.uint16(0x7F00)


def test_nvfp4_hand_examples():
    # tensor scale 1: block scale = e4m3(amax / 6)
    x = _bf([[6.0, 2.703125] + [0.0] * 14 +            # b = 1: 2.703 -> 3
             [12.0, 5.0, -3.0] + [0.0] * 13 +          # b = 2: 2.5 -> 2 -> 4; -1.5 -> -3
             [6.5, 1.0] + [0.0] * 14 +                 # b = e4m3(1.0833) = 1.125: 5.78 -> 6
             [0.0] * 16])
    out, b = oracle.fake_quant_nvfp4(x, 1.0)
    np.testing.assert_array_equal(b, [[1.0, 2.0, 1.125, 0.0]])
    got = bf16_bits_to_f32(out)[0]
    np.testing.assert_array_equal(got[:2], [6.0, 3.0])
    np.testing.assert_array_equal(got[16:19], [12.0, 4.0, -3.0])
    # 6.5 / 1.125 = 5.78 -> 6 -> 6.75; 1 / 1.125 = 0.889 -> 1 -> 1.125
    np.testing.assert_array_equal(got[32:34], [6.75, 1.125])
    assert np.all(out[0, 48:] == 0)
    # a zero tensor scale zeroes everything
    out0, _ = oracle.fake_quant_nvfp4(x, 0.0)
    assert np.all(out0 == 0)


def test_nvfp4_tensor_scale_closed_form():
    assert oracle.nvfp4_tensor_scale(6 * 448) == np.float32(1.0)
    assert oracle.nvfp4_tensor_scale(0) == np.float32(0.0)


def test_fp4_row_mask_leaves_rows():
    rng = np.random.default_rng(3)
    x = _bf(rng.standard_normal((4, 64)))
    mask = np.array([True, False, True, False])
    for fn in (lambda a, m: oracle.fake_quant_mxfp4(a, m),
               lambda a, m: oracle.fake_quant_nvfp4(a, 0.01, m)):
        out, sc = fn(x, mask)
        np.testing.assert_array_equal(out[~mask], x[~mask])
        assert np.all(sc[~mask] == 0)
        assert not np.array_equal(out[mask], x[mask])


def test_fp8_weight_blocks_hand_examples():
    """Weights in E4M3 with one scale per 128x128 tile: tile (0, 1) has amax
    448 (scale 1, E4M3 step 0.25 in [2, 4): 3.09375 -> 3), tile (1, 0) amax
    4.48 -> bf16 4.46875, scale fl32(4.46875/448); tile (1, 1) is all zero."""
    w = np.zeros((256, 256), np.float32)
    w[5, 130] = 448.0
    w[7, 200] = 3.09375
    w[7, 201] = -3.15625                       # nearer to -3.25 than to -3
    w[140, 3] = 4.46875
    w[141, 4] = -4.46875
    q, s, deq = oracle.quantize_weight_blocks(f32_to_bf16_bits(w))
    s_10 = np.float32(np.float32(4.46875) / np.float32(448))
    np.testing.assert_array_equal(s, np.array([[0, 1], [s_10, 0]], np.float32))
    assert q[7, 200] == 3.0 and q[7, 201] == -3.25 and q[5, 130] == 448.0
    assert abs(q[140, 3]) == 448.0 and q[141, 4] == -q[140, 3]
    d = bf16_bits_to_f32(deq)
    assert d[7, 200] == 3.0 and d[7, 201] == -3.25 and d[5, 130] == 448.0
    assert d[140, 3] == np.float32(4.46875)    # 448 * s rounds back to the bf16 amax
    assert np.count_nonzero(d) == 5
