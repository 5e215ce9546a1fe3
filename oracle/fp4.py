"""Oracle for the FP4 fake-quantizers (MXFP4 and NVFP4) — test infrastructure
only (see the package docstring).

Sources: "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM
Mega-MoE" names NVFP4 dispatch and combine units (the usage section and
"Testing": an NVFP4 dispatch + combine setup); "[Bugfix][MoE] Size the
permute scratch from its inputs" runs an MXFP4 expert path in its test
plan.  Neither page defines the formats, so the definitions below are the
published ones (readings, listed with the others in the design notes):

* E2M1 (the FP4 element of both): 1 sign, 2 exponent bits (bias 1), 1
  mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Round to nearest,
  ties to the even code (last mantissa bit 0), saturating at 6.
* MXFP4 (OCP Microscaling): blocks of 32 consecutive channels of a row; the
  shared scale is the power of two ``X = 2^(floor(log2(amax)) - 2)``
  (2 = the largest E2M1 exponent), its exponent clamped to the E8M0 range
  [-127, 127]; element ``e2m1(x / X)``; an all-zero block stays +0.
  Output ``bf16(e2m1 * X)`` (exact: few significant bits times a power of 2).
* NVFP4: blocks of 16 channels; a float32 per-tensor scale ``g`` (given,
  like the FP8 combine scale: calibrated or constant) and an E4M3 block
  scale ``b = e4m3(min(fl32(amax / fl32(6 g)), 448))``; with
  ``S = fl32(b * g)``: ``x' = bf16(fl32(e2m1(clamp(fl32(x / S), +-6)) * S))``;
  ``S == 0`` gives a block of +0.

Every ``fl32`` is one IEEE binary32 operation (numpy float32 arithmetic).
"""

import numpy as np

from .numerics import bf16_bits_to_f32, f32_to_bf16_bits, e4m3fn_round, E4M3FN_MAX

E2M1_MAX = 6.0


def e2m1_table() -> np.ndarray:
    """Magnitudes of the 8 non-negative E2M1 codes, in code order (also
    ascending value order): code = (exponent << 1) | mantissa."""
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        vals.append(m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return np.array(vals, dtype=np.float64)


_E2M1 = e2m1_table()


def e2m1_round(v) -> np.ndarray:
    """Nearest E2M1 value to each ``v`` with ``|v| <= 6`` (ties to the even
    code).  Returns exact float64 values with the sign of ``v``."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E2M1_MAX) or np.any(np.isnan(a)):
        raise ValueError("e2m1_round expects finite values within +-6")
    d = np.abs(a[..., None] - _E2M1)                       # distance to every code
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                       # one or two nearest codes
    codes = np.arange(8)
    # among the nearest codes prefer the even one (a tie has one of each)
    pick = np.where(cand & (codes % 2 == 0), codes, 99).min(axis=-1)
    pick = np.where(pick == 99, np.where(cand, codes, 99).min(axis=-1), pick)
    return np.copysign(_E2M1[pick], v)


def _blocks(x_bits, block):
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, H = x_bits.shape
    if H % block:
        raise ValueError("H must be a multiple of the block size")
    return x_bits, bf16_bits_to_f32(x_bits).reshape(R, H // block, block)


def _restore(out, x_bits, row_mask, scales):
    if row_mask is not None:
        keep = ~np.asarray(row_mask, dtype=bool)
        out[keep] = x_bits[keep]
        scales = scales.copy()
        scales[keep] = 0
    return out, scales


def fake_quant_mxfp4(x_bits, row_mask=None):
    """MXFP4 fake-quant of bfloat16 rows [R, H] (H a multiple of 32).

    Returns ``(out_bits uint16 [R, H], scales float64 [R, H/32])`` with the
    shared power-of-two scale of each block (0 for all-zero blocks and for
    rows where ``row_mask`` is False, which are returned unchanged)."""
    x_bits, x = _blocks(x_bits, 32)
    amax = np.abs(x).max(axis=2).astype(np.float64)
    nz = amax > 0
    _, e = np.frexp(np.where(nz, amax, 1.0))               # amax = m 2^e, m in [0.5, 1)
    xexp = np.clip(e - 1 - 2, -127, 127)
    X = np.where(nz, np.ldexp(1.0, xexp), 0.0)
    r = np.where(nz[..., None], x.astype(np.float64) / np.where(nz, X, 1.0)[..., None], 0.0)
    q = e2m1_round(np.clip(r, -E2M1_MAX, E2M1_MAX))
    vals = q * X[..., None]                                # exact
    out = f32_to_bf16_bits(vals.astype(np.float32)).reshape(x_bits.shape)
    out = np.where(np.repeat(nz, 32, axis=1).reshape(x_bits.shape), out, np.uint16(0))
    return _restore(out.astype(np.uint16), x_bits, row_mask, X)


def fake_quant_nvfp4(x_bits, g, row_mask=None):
    """NVFP4 fake-quant of bfloat16 rows [R, H] (H a multiple of 16) with the
    float32 per-tensor scale ``g``.

    Returns ``(out_bits uint16 [R, H], block_scales float64 [R, H/16])`` with
    the E4M3 block scale ``b`` of each block (0 for rows where ``row_mask`` is
    False, which are returned unchanged)."""
    x_bits, x = _blocks(x_bits, 16)
    g = np.float32(g)
    amax = np.abs(x).max(axis=2)                           # float32, exact
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (amax / np.float32(np.float32(6.0) * g)).astype(np.float32)
    q = np.where(np.isnan(q), np.float32(0), q)            # 0 / 0: an all-zero block
    b = e4m3fn_round(np.minimum(q.astype(np.float64), E4M3FN_MAX))
    S = (b.astype(np.float32) * g).astype(np.float32)
    safe = np.where(S > 0, S, np.float32(1))
    with np.errstate(over="ignore"):                       # +-inf saturates to +-6 below
        r = (x / safe[..., None]).astype(np.float32)
    e = e2m1_round(np.clip(r.astype(np.float64), -E2M1_MAX, E2M1_MAX))
    vals = (e.astype(np.float32) * S[..., None]).astype(np.float32)
    out = f32_to_bf16_bits(vals).reshape(x_bits.shape)
    zero = np.repeat(S <= 0, 16, axis=1).reshape(x_bits.shape)
    out = np.where(zero, np.uint16(0), out).astype(np.uint16)
    return _restore(out, x_bits, row_mask, b)


def nvfp4_tensor_scale(amax) -> np.float32:
    """The per-tensor NVFP4 scale from a calibrated amax: ``fl32(amax / fl32(6 * 448))``."""
    return np.float32(np.float32(amax) / np.float32(np.float32(6.0) * np.float32(E4M3FN_MAX)))
