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
