"""Helpers for the GPU parity tests: numpy <-> device tensors, seeded inputs.

bfloat16 data travels as uint16 bit patterns on the host and as
torch.bfloat16 on the device (same bits).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def stacked_weights(cfg: workloads.MoEConfig, experts=None):
    """All experts' weights on the device as [E, 2I, H] and [E, H, I] bf16,
    plus a host dict expert -> (w13, w2) bit arrays for the oracle."""
    experts = list(range(cfg.E)) if experts is None else list(experts)
    w13 = torch.empty(len(experts), 2 * cfg.I, cfg.H, dtype=torch.bfloat16, device="cuda")
    w2 = torch.empty(len(experts), cfg.H, cfg.I, dtype=torch.bfloat16, device="cuda")
    host_w = {}
    pos = {e: i for i, e in enumerate(experts)}

    def put(e, a, b):
        w13[pos[e]] = dev_bf16(a)
        w2[pos[e]] = dev_bf16(b)
        host_w[e] = (a, b)

    workloads.for_each_expert(cfg, put, experts)
    return w13, w2, host_w


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def check_rows(got, ref, tol: float = 2e-2, what: str = "") -> dict:
    """Three bounds on a [rows, H] result against its reference, all at the
    FFN tolerance ``tol``:

    * the Frobenius relative error over all rows;
    * every row's relative error ``||got_r - ref_r|| / ||ref_r||`` (a row
      whose reference is all zero must come out within ``tol`` times the
      largest reference magnitude);
    * every element: ``|got - ref| <= tol * max|ref_r|`` of its row.

    A wrong 16 x 16 output tile, a few wrong rows or a single wrong element
    fails the second or third bound even when the norm over a large batch
    barely moves.  Returns the three measured figures."""
    got = np.asarray(got, dtype=np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    frob = rel_err(got, ref)
    if got.size == 0:
        return {"frob": 0.0, "worst_row": 0.0, "worst_elem": 0.0}
    diff = got - ref
    rn = np.linalg.norm(ref, axis=1)
    scale_all = max(float(np.abs(ref).max()), 1e-30)
    row_err = np.where(rn > 0, np.linalg.norm(diff, axis=1) / np.where(rn > 0, rn, 1.0),
                       np.abs(got).max(axis=1) / scale_all)
    rmax = np.abs(ref).max(axis=1)
    elem = np.abs(diff).max(axis=1) / np.where(rmax > 0, rmax, scale_all)
    out = {"frob": frob, "worst_row": float(row_err.max()), "worst_elem": float(elem.max())}
    assert frob <= tol, (what, "frobenius", out)
    assert out["worst_row"] <= tol, (what, "row", int(row_err.argmax()), out)
    assert out["worst_elem"] <= tol, (what, "element", int(elem.argmax()), out)
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN bytes to values (sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent 0 subnormal).  NaN codes must not appear."""
    c = np.asarray(codes).astype(np.int64)
    assert not np.any((c & 0x7F) == 0x7F), "NaN code"
    e, m = (c >> 3) & 0xF, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.where(c & 0x80, -mag, mag)


def w8a8_intermediate(ws: torch.Tensor, capacity: int, G: int, I: int, counts, cu_seqlens):
    """The FP8 path's intermediate ``a`` as moe_grouped_ffn_w8a8's gate/up
    stage leaves it in its workspace, decoded to per-row values: codes
    (float64 E4M3 values) [capacity, I] and scales [capacity, I/128], indexed
    by permuted row.  The workspace layout (the down GEMM's operand order,
    per 128-row m-tile of each segment, m-tiles numbered over the segments in
    order): 16-byte unit ((((m*8 + i)*nkb + kb)*2 + h)*64 + l), lane
    l = row%16 + 16*g, byte b, holds row 16 i + row%16 of m-tile m, column
    128 kb + 64 h + 16 g + b; then the scales, float32
    [m-tile][I/128][128 rows]."""
    m_tiles = (capacity + 127) // 128 + G
    nkb = I // 128
    raw = ws.cpu().numpy().view(np.uint8)
    nbytes = m_tiles * 128 * I
    codes = raw[:nbytes].reshape(m_tiles, 8, nkb, 2, 4, 16, 16)      # m i kb h g r b
    codes = codes.transpose(0, 1, 5, 2, 3, 4, 6).reshape(m_tiles * 128, I)
    off = (nbytes + 255) & ~255
    sc = raw[off:off + m_tiles * nkb * 128 * 4].view(np.float32).reshape(m_tiles, nkb, 128)
    sc = sc.transpose(0, 2, 1).reshape(m_tiles * 128, nkb)
    qa = np.zeros((capacity, I))
    sa = np.zeros((capacity, nkb), np.float32)
    mt0 = 0
    for g in range(G):
        n, r0 = int(counts[g]), int(cu_seqlens[g])
        if n:
            qa[r0:r0 + n] = e4m3_decode(codes[mt0 * 128:mt0 * 128 + n])
            sa[r0:r0 + n] = sc[mt0 * 128:mt0 * 128 + n]
        mt0 += (n + 127) // 128
    return qa, sa


def check_fp8_intermediate(qa_gpu, sa_gpu, qa_ref, sa_ref, what: str = "") -> float:
    """The GPU's intermediate codes against the oracle's: the same E4M3 code
    and scale almost everywhere.  ``a`` comes from a float32 accumulation on
    the GPU and a float64 one in the oracle, which differ by a few 1e-6 of
    the block's largest products (float32 rounding over a K of a few hundred
    to a few thousand terms), so:

    * a block scale may differ where its amax rounds to the neighbouring
      bf16 value: by one bf16 ulp (2^-8 relative), in at most 5 % of blocks;
    * a code may differ where the value crosses an E4M3 rounding boundary:
      by at most one E4M3 step of the value, plus 2^-4 code units (2^-4 / 448
      of the block's amax) for the smallest values, where that absolute
      difference spans several subnormal steps; in at most 2 % of elements.

    A wrong layout, a row or column mix-up or a wrong scale breaks these for
    most elements.  Returns the fraction of differing codes."""
    qa_gpu, qa_ref = np.asarray(qa_gpu), np.asarray(qa_ref)
    sa_gpu, sa_ref = np.asarray(sa_gpu, np.float64), np.asarray(sa_ref, np.float64)
    s_diff = sa_gpu != sa_ref
    rel = np.abs(sa_gpu - sa_ref) / np.where(sa_ref > 0, sa_ref, 1.0)
    if s_diff.mean() > 0.05 or np.any(rel > 2.0 ** -7):
        r, c = np.nonzero(s_diff)
        info = [(int(a), int(b), float(sa_gpu[a, b]), float(sa_ref[a, b])) for a, b in zip(r[:12], c[:12])]
        raise AssertionError((what, "scales", float(s_diff.mean()), float(rel.max()), info))
    same_scale = np.repeat(~s_diff, 128, axis=1)
    diff = (qa_gpu != qa_ref) & same_scale
    frac = float(diff.mean())
    a, b = np.abs(qa_gpu[diff]), np.abs(qa_ref[diff])
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.maximum(a, b), 2.0 ** -6))) - 3)
    bad = np.abs(qa_gpu[diff] - qa_ref[diff]) > step + 2.0 ** -4
    if frac > 0.02 or bad.any():
        rows, cols = np.nonzero(diff)
        sel = np.nonzero(bad)[0][:12] if bad.any() else np.arange(min(12, len(rows)))
        info = [(int(rows[k]), int(cols[k]), float(qa_gpu[rows[k], cols[k]]),
                 float(qa_ref[rows[k], cols[k]]), float(sa_gpu[rows[k], cols[k] // 128]))
                for k in sel]
        raise AssertionError((what, "codes", frac, int(bad.sum()), info))
    return frac
