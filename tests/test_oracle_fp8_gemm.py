"""Pins for the real-FP8 FFN oracle (CPU only).

* quantize_rows_fp8 is the dispatch fake-quant's quantizer: dequantizing its
  codes with its scales gives fake_quant_block's output bit for bit (that
  one is pinned exhaustively against torch's float8_e4m3fn), and its codes
  are exactly E4M3 values.
* block_scaled_matmul against a scalar triple loop on tiny inputs with a
  different scale on every block and tile (a transposed or misindexed scale
  fails it).
* expert_ffn_w8a8 on inputs that quantize exactly (every block's amax is
  448 times a power of two and every value a code times that scale): its
  only error against the float64 expert_ffn is the rounding of the
  intermediate ``a`` to bfloat16 and to E4M3, which is bounded element by
  element.
"""

import numpy as np

import oracle
from oracle.fp8_gemm import block_scaled_matmul, expert_ffn_w8a8, quantize_rows_fp8
from oracle.numerics import bf16_bits_to_f32, f32_to_bf16_bits

def _rows(R, H, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((R, H)) * np.exp2(rng.integers(-6, 6, (R, 1)))).astype(np.float32)
    x[1, 128:256] = 0.0                                   # an all-zero block
    x[2, 5] = 1e-30                                       # below every E4M3 step
    return f32_to_bf16_bits(x)


def test_quantize_rows_matches_fake_quant():
    xb = _rows(6, 384, 1)
    mask = np.array([1, 1, 1, 0, 1, 1], bool)
    q, s = quantize_rows_fp8(xb, row_mask=mask)
    fq, fs = oracle.fake_quant_block(xb, 128, row_mask=mask)
    np.testing.assert_array_equal(s.view(np.uint32), fs.view(np.uint32))
    deq = f32_to_bf16_bits((q.reshape(6, 3, 128) * s[:, :, None].astype(np.float64))
                           .astype(np.float32).reshape(6, 384))
    np.testing.assert_array_equal(deq[mask], fq[mask])
    assert np.all(q[~mask] == 0) and np.all(s[~mask] == 0)
    assert np.all(q[1, 128:256] == 0) and s[1, 1] == 0
    table = set(np.abs(oracle.e4m3fn_table()).tolist())
    assert set(np.unique(np.abs(q)).tolist()) <= table


def test_block_scaled_matmul_brute_force():
    rng = np.random.default_rng(2)
    M, N, K = 3, 256, 256
    tab = oracle.e4m3fn_table()
    tab = tab[np.isfinite(tab)]
    qa = rng.choice(tab, (M, K))
    qb = rng.choice(tab, (N, K))
    sa = rng.uniform(0.5, 2.0, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.5, 2.0, (N // 128, K // 128)).astype(np.float32)
    got = block_scaled_matmul(qa, sa, qb, sb)
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(sa[m, k // 128]) * float(sb[n // 128, k // 128]) * qa[m, k] * qb[n, k]
            want[m, n] = acc
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-9)


def _exact_fp8(shape, block_shape, rng):
    """Values that quantize exactly: per block a power-of-two scale s, codes
    drawn from the E4M3 grid with one element of the block at +-448 (so the
    block's amax is exactly 448 s)."""
    tab = oracle.e4m3fn_table()
    tab = tab[np.isfinite(tab) & (np.abs(tab) <= 448)]
    q = rng.choice(tab, shape)
    R, C = shape
    br, bc = block_shape
    scale = np.exp2(rng.integers(-12, -6, (R // br, C // bc))).astype(np.float64)
    for i in range(R // br):
        for j in range(C // bc):
            q[i * br, j * bc] = 448.0 * rng.choice([-1.0, 1.0])
    return q * np.repeat(np.repeat(scale, br, 0), bc, 1)


def test_expert_ffn_w8a8_error_is_the_intermediate_rounding():
    rng = np.random.default_rng(3)
    n, H, I = 5, 256, 128
    x = _exact_fp8((n, H), (1, 128), rng)
    w13 = _exact_fp8((2 * I, H), (128, 128), rng)
    w2 = _exact_fp8((H, I), (128, 128), rng)
    xb, w13b, w2b = (f32_to_bf16_bits(v.astype(np.float32)) for v in (x, w13, w2))
    assert np.array_equal(bf16_bits_to_f32(xb), x.astype(np.float32))     # bf16-exact inputs
    qx, sx = quantize_rows_fp8(xb)
    got = expert_ffn_w8a8(qx, sx, w13b, w2b)
    # exact gate/up on exactly quantized inputs, then the bound on a's roundings
    h = x @ w13.T
    a = oracle.ffn.silu(h[:, :I]) * h[:, I:]
    want = a @ w2.T
    amax = np.abs(a).reshape(n, I // 128, 128).max(axis=2)
    s_a = np.repeat(amax / 448.0, 128, axis=1) * (1 + 2.0 ** -8)
    da = np.maximum(2.0 ** -4 * np.abs(a), 2.0 ** -10 * s_a) * (1 + 2.0 ** -7) + 2.0 ** -8 * np.abs(a)
    bound = da @ np.abs(w2).T + 1e-12
    assert np.all(np.abs(got - want) <= bound)
    # and the bound is not vacuous: a dropped block scale breaks it
    qa_bad = expert_ffn_w8a8(qx, sx * np.float32(2), w13b, w2b)
    assert not np.all(np.abs(qa_bad - want) <= bound)


def test_grouped_ffn_w8a8_equals_row_by_row():
    """The segment loop against each row computed on its own: hand-built
    segments with an empty expert and pow2 padding rows (garbage codes that
    must not be computed), a different router weight per row.  A wrong
    segment start, a slice of the wrong expert's weights or router weights,
    or padding rows that leak into the output fail it."""
    rng = np.random.default_rng(21)
    H, I = 256, 128
    counts = np.array([3, 0, 5, 1], np.int32)
    sizes = np.array([4, 0, 8, 1])                        # next powers of two
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    cap = int(cu[-1])
    xb = _rows(cap, H, 22)
    qx, sx = quantize_rows_fp8(xb)
    valid = np.zeros(cap, bool)
    for e in range(4):
        valid[cu[e]:cu[e] + counts[e]] = True
    qx[~valid] = 448.0                                    # padding rows hold garbage
    sx[~valid] = np.float32(1e3)
    w = {e: (f32_to_bf16_bits((rng.standard_normal((2 * I, H)) * 0.05).astype(np.float32)),
             f32_to_bf16_bits((rng.standard_normal((H, I)) * 0.05).astype(np.float32)))
         for e in range(4)}
    row_scale = rng.uniform(0.1, 1.0, cap).astype(np.float32)
    got = oracle.grouped_ffn_w8a8(qx, sx, cu, counts, lambda e: w[e], row_scale)
    assert np.all(got[~valid] == 0)
    for e in range(4):
        for r in range(cu[e], cu[e] + counts[e]):
            want = expert_ffn_w8a8(qx[r:r + 1], sx[r:r + 1], *w[e])[0] * float(row_scale[r])
            np.testing.assert_allclose(got[r], want, rtol=1e-9, atol=1e-12)
