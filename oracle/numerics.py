"""Number formats used by the oracle: bfloat16 and OCP FP8 E4M3FN.

Test infrastructure only (see the package docstring).

Both roundings are written from the format definitions, as "pick the nearest
representable value, ties to the one whose last mantissa bit is 0", by
enumerating the two candidate neighbours and comparing distances in float64
(where every distance here is exact).  They are pinned against torch's CPU
casts, which are an independent implementation of the same IEEE / OCP rules.

Sources:
* "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM Mega-MoE",
  PR summary and "How it works": the combine ends in one BF16 rounding; the
  quantizers are FP8 fake-quantizers (quantize then dequantize).
* The configurations fix the FP8 flavour as e4m3 with scale amax/448, i.e.
  the OCP E4M3FN format (max finite 448, no infinities).
"""

import numpy as np

# ---------------------------------------------------------------------------
# bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits.
# Storage convention everywhere: the 16-bit pattern as numpy uint16.
# ---------------------------------------------------------------------------


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def _bf16_ulp_above(trunc_bits: np.ndarray) -> np.ndarray:
    """Magnitude of one bfloat16 ulp for a truncated pattern (float64, exact)."""
    exp_field = ((trunc_bits >> np.uint64(23)) & np.uint64(0xFF)).astype(np.int64)
    # subnormals (exp field 0) share the spacing of the smallest normal binade
    e = np.maximum(exp_field, 1) - 127 - 7
    return np.ldexp(np.ones(e.shape, dtype=np.float64), e)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest, ties-to-even.

    Candidates: ``lo`` = x with the low 16 bits dropped (same sign, not larger
    in magnitude) and ``hi`` = the next bfloat16 away from zero (for the
    largest finite value that is +-inf, which IEEE treats as 2^128 for the
    purpose of rounding).  The nearer one wins; on a tie the one with an even
    last mantissa bit wins.  NaN maps to the quiet NaN 0x7FC0 (sign kept);
    infinities stay infinities.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    sign = bits & np.uint64(0x80000000)
    mag = bits & np.uint64(0x7FFFFFFF)
    is_nan = mag > np.uint64(0x7F800000)
    is_inf = mag == np.uint64(0x7F800000)

    lo_mag = mag & np.uint64(0x7FFF0000)
    hi_mag = lo_mag + np.uint64(0x10000)
    lo_val = (lo_mag.astype(np.uint32)).view(np.float32).astype(np.float64)
    hi_val = lo_val + _bf16_ulp_above(lo_mag)
    xv = np.abs(x.astype(np.float64))
    with np.errstate(invalid="ignore"):              # inf/NaN lanes are overwritten below
        d_lo = xv - lo_val
        d_hi = hi_val - xv
    lo_is_odd = ((lo_mag >> np.uint64(16)) & np.uint64(1)) == np.uint64(1)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & lo_is_odd)
    take_hi &= d_lo != 0.0
    out_mag = np.where(take_hi, hi_mag, lo_mag) >> np.uint64(16)
    out = (sign >> np.uint64(16)) | out_mag
    out = np.where(is_inf, (sign >> np.uint64(16)) | np.uint64(0x7F80), out)
    out = np.where(is_nan, (sign >> np.uint64(16)) | np.uint64(0x7FC0), out)
    return out.astype(np.uint16)


# ---------------------------------------------------------------------------
# OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
# Codes with exponent field 0 are subnormal (m * 2^-9); 0x7F / 0xFF are NaN;
# there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
# ---------------------------------------------------------------------------

E4M3FN_MAX = 448.0


def e4m3fn_table() -> np.ndarray:
    """Values of the 127 non-negative finite codes 0x00..0x7E, in code order.

    Code order is also ascending value order, so the table is sorted.
    """
    vals = []
    for code in range(0x7F):
        e = code >> 3
        m = code & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


_TABLE = e4m3fn_table()


def e4m3fn_round(v) -> np.ndarray:
    """Nearest E4M3FN value to each finite ``v`` with ``|v| <= 448``.

    Round-to-nearest with ties to the even code (last mantissa bit 0).  Input
    outside [-448, 448] is a caller error (the fake-quantizer clamps first),
    so this function never meets the NaN codes.  Returns exact float64 values.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3FN_MAX) or np.any(np.isnan(a)):
        raise ValueError("e4m3fn_round expects finite values within +-448")
    hi_idx = np.searchsorted(_TABLE, a, side="left")      # first value >= a
    hi_idx = np.minimum(hi_idx, len(_TABLE) - 1)
    lo_idx = np.maximum(hi_idx - 1, 0)
    exact = _TABLE[hi_idx] == a
    lo_val = _TABLE[lo_idx]
    hi_val = _TABLE[hi_idx]
    d_lo = a - lo_val
    d_hi = hi_val - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo_idx & 1) == 1))
    mag = np.where(exact | take_hi, hi_val, lo_val)
    return np.copysign(mag, v)


def qdq_e4m3fn(x_f32, s_f32) -> np.ndarray:
    """Fake-quantize float32 values with a float32 scale to bfloat16 bits.

    ``x' = bf16( fl32( e4m3( clamp(fl32(x / s), -448, 448) ) * s ) )``.
    Each ``fl32`` is one correctly rounded binary32 operation (numpy float32
    division and multiplication are IEEE).  ``s`` broadcasts against ``x``.
    Where ``s == 0`` (an all-zero block) the output is +0.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    s = np.asarray(s_f32, dtype=np.float32)
    s_b = np.broadcast_to(s, x.shape)
    zero = s_b == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        ratio = np.where(zero, np.float32(0), x / np.where(zero, np.float32(1), s_b))
    ratio = np.clip(ratio.astype(np.float32), np.float32(-E4M3FN_MAX), np.float32(E4M3FN_MAX))
    q = e4m3fn_round(ratio).astype(np.float32)          # exact: e4m3 values fit in binary32
    deq = (q * s_b).astype(np.float32)                   # one binary32 rounding
    out = f32_to_bf16_bits(deq)
    return np.where(zero, np.uint16(0), out).astype(np.uint16)
