"""Pins of the oracle's stages: brute force, closed forms, hand examples.

Each test checks the oracle against something other than itself, so that a
dropped term, a wrong index or sign, or a swapped operand fails here.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle.numerics import bf16_bits_to_f32, f32_to_bf16_bits
from oracle.ffn import silu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------- route

def _brute_topk(row, k):
    """The unique k-subset whose members all beat all non-members, where a
    beats b iff (value_a > value_b) or (equal values and a < b)."""
    E = len(row)
    beats = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
    found = []
    for S in itertools.combinations(range(E), k):
        rest = [j for j in range(E) if j not in S]
        if all(beats(a, b) for a in S for b in rest):
            found.append(S)
    assert len(found) == 1
    S = list(found[0])
    # order inside the subset by the same relation (insertion sort)
    out = []
    for a in S:
        pos = 0
        while pos < len(out) and beats(out[pos], a):
            pos += 1
        out.insert(pos, a)
    return out


@pytest.mark.parametrize("k", [1, 2, 3])
def test_route_topk_matches_subset_enumeration_with_ties(k):
    rng = np.random.default_rng(10 + k)
    # small integers force many ties; -0.0 and 0.0 compare equal
    logits = rng.integers(-2, 3, size=(16, 8)).astype(np.float32)
    logits[0, :] = 0.0
    logits[1, ::2] = -0.0
    idx, w = oracle.route(logits, None, k)
    for t in range(16):
        assert list(idx[t]) == _brute_topk(logits[t], k)


def test_route_closed_form_weights():
    logits = np.array([[0.0, math.log(2.0), math.log(3.0)]], dtype=np.float32)
    idx, w = oracle.route(logits, None, 2)
    assert list(idx[0]) == [2, 1]
    np.testing.assert_allclose(w[0], [0.6, 0.4], rtol=1e-6)
    # without renormalisation: plain softmax entries 3/6 and 2/6
    idx, w = oracle.route(logits, None, 2, renormalize=False)
    np.testing.assert_allclose(w[0], [0.5, 1 / 3], rtol=1e-6)


def test_route_full_k_without_renorm_is_softmax():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((32, 6)).astype(np.float32)
    idx, w = oracle.route(logits, None, 6, renormalize=False)
    sm = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(sm, idx, axis=1), rtol=1e-6)


def test_route_invariants_and_padding():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((50, 16)).astype(np.float32)
    valid = (rng.random(50) > 0.2).astype(np.uint8)
    idx, w = oracle.route(logits, valid, 4)
    for t in range(50):
        if not valid[t]:
            assert np.all(idx[t] == -1) and np.all(w[t] == 0)
            continue
        sel = logits[t, idx[t]]
        assert np.all(np.diff(sel) <= 0)                 # slot 0 is the largest
        assert len(set(idx[t])) == 4
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 1e-6
        assert np.all(np.diff(w[t]) <= 0)


def test_route_nan_ranks_as_minus_infinity():
    """A NaN logit ranks exactly like -inf (below every number, ties among
    such entries to the lower index), checked against the brute-force
    subset order on the row with -inf written in; weights against closed
    forms: a chosen -inf below a finite maximum weighs 0, and a row whose
    chosen logits are all -inf (or NaN) splits 1/k evenly."""
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    logits = np.array([
        [nan, 1.0, 0.5, nan, 2.0, -3.0],       # NaNs among finite values
        [nan, nan, nan, nan, nan, nan],        # all NaN
        [-inf, nan, 0.0, -inf, nan, -1.0],     # fewer than k finite
        [inf, 1.0, inf, nan, -inf, 0.0],       # two +inf: they tie at the top
    ], dtype=np.float32)
    k = 3
    idx, w = oracle.route(logits, None, k)
    as_inf = np.where(np.isnan(logits), -inf, logits)
    for t in range(len(logits)):
        assert list(idx[t]) == _brute_topk(as_inf[t], k), t
    np.testing.assert_allclose(w[0], scipy.special.softmax([2.0, 1.0, 0.5]), rtol=1e-6)
    assert list(idx[1]) == [0, 1, 2] and np.all(w[1] == np.float32(1 / 3))
    assert list(idx[2]) == [2, 5, 0]
    np.testing.assert_allclose(w[2], [1 / (1 + math.exp(-1)), math.exp(-1) / (1 + math.exp(-1)), 0.0],
                               rtol=1e-6)
    assert list(idx[3]) == [0, 2, 1] and list(w[3]) == [0.5, 0.5, 0.0]
    # without renormalisation the denominator runs over all E the same way
    _, w_full = oracle.route(logits, None, k, renormalize=False)
    np.testing.assert_allclose(w_full[0], scipy.special.softmax([2.0, 1.0, 0.5, -3.0])[:3],
                               rtol=1e-6)
    assert np.all(w_full[1] == np.float32(1 / 6))


# ----------------------------------------------------------------- fake quant

def test_block_fake_quant_blocks_are_independent():
    rng = np.random.default_rng(5)
    x = f32_to_bf16_bits(rng.standard_normal((6, 256)).astype(np.float32))
    x[2, 128:] = 0                                       # an all-zero block
    out, s = oracle.fake_quant_block(x, 128)
    for r in range(6):
        for b in range(2):
            blk = bf16_bits_to_f32(x[r, b * 128:(b + 1) * 128])
            amax = np.float32(np.abs(blk).max())
            assert s[r, b] == np.float32(amax / np.float32(448))
            want = oracle.qdq_e4m3fn(blk, s[r, b]) if amax > 0 else np.zeros(128, np.uint16)
            np.testing.assert_array_equal(out[r, b * 128:(b + 1) * 128], want)
    # a masked (padding) row passes through untouched
    out2, s2 = oracle.fake_quant_block(x, 128, row_mask=np.array([1, 1, 1, 1, 1, 0], bool))
    np.testing.assert_array_equal(out2[5], x[5])
    assert np.all(s2[5] == 0)


def test_calibrated_amax_is_max_abs():
    x = f32_to_bf16_bits(np.array([[1.5, -7.25], [3.0, 0.5]], np.float32))
    assert oracle.calibrate_amax(x) == np.float32(7.25)
    assert oracle.calibrate_amax(x, np.array([False, True])) == np.float32(3.0)


# -------------------------------------------------------------------- permute

def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_permute_hand_examples():
    for case in _load("permute_small.json")["cases"]:
        idx = np.array(case["topk_idx"], dtype=np.int32)
        T, K = idx.shape
        w = np.arange(T * K, dtype=np.float32).reshape(T, K) + 1
        hid = np.arange(T * 4, dtype=np.uint16).reshape(T, 4)
        p = oracle.permute(idx, w, hid, case["E"], case["expert_begin"], case["pad_pow2"])
        for key in ("counts", "cu_seqlens", "row_of", "src_of"):
            assert p[key].tolist() == case[key], key


def test_permute_expert_ids_past_the_layer_are_reported_not_routed():
    """An id at or past the layer's expert count is dropped and reported;
    the other slots land exactly where they would without it; negative ids
    of any value are padding slots (not reported)."""
    idx = np.array([[0, 9], [3, -1], [-5, 2], [4, 1]], np.int32)   # E = 5: 9 is bad
    w = np.arange(8, dtype=np.float32).reshape(4, 2) + 1
    hid = np.arange(16, dtype=np.uint16).reshape(4, 4)
    p = oracle.permute(idx, w, hid, 5, num_experts=5)
    assert p["expert_range_error"]
    assert p["row_of"].tolist() == [0, -1, 3, -1, -1, 2, 4, 1]
    assert p["counts"].tolist() == [1, 1, 1, 1, 1]
    clean = idx.copy()
    clean[0, 1] = -1
    q = oracle.permute(clean, w, hid, 5, num_experts=5)
    assert not q["expert_range_error"]
    for key in ("counts", "cu_seqlens", "row_of", "src_of", "w_perm", "x_perm"):
        np.testing.assert_array_equal(p[key], q[key])
    # an expert-parallel share of [2, 4) inside 5 experts: 4 belongs to
    # another rank (not reported), 9 to none (reported)
    r = oracle.permute(idx, w, hid, 2, expert_begin=2, num_experts=5)
    assert r["expert_range_error"] and r["counts"].tolist() == [1, 1]


def _permute_by_stable_argsort(idx, El, expert_begin):
    """Non-pow2 permute via numpy's stable argsort of the expert keys."""
    flat = idx.reshape(-1).astype(np.int64) - expert_begin
    routed = (idx.reshape(-1) >= 0) & (flat >= 0) & (flat < El)
    key = np.where(routed, flat, El)                     # unrouted sort last
    order = np.argsort(key, kind="stable")
    n = int(routed.sum())
    src_of = order[:n].astype(np.int32)
    row_of = np.full(idx.size, -1, np.int32)
    row_of[src_of] = np.arange(n, dtype=np.int32)
    return src_of, row_of


@pytest.mark.parametrize("seed", range(6))
def test_permute_matches_stable_argsort_and_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    T, K, E = int(rng.integers(1, 40)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    hid = rng.integers(0, 2**16, size=(T, 8), dtype=np.uint64).astype(np.uint16)
    begin = int(rng.integers(0, max(E - 1, 1)))
    El = int(rng.integers(1, E - begin + 1))
    p = oracle.permute(idx, w, hid, El, begin, pad_pow2=False)
    src_of, row_of = _permute_by_stable_argsort(idx, El, begin)
    np.testing.assert_array_equal(p["src_of"], src_of)
    np.testing.assert_array_equal(p["row_of"], row_of)

    # power-of-two mode: same valid rows per segment, shifted by padding
    q = oracle.permute(idx, w, hid, El, begin, pad_pow2=True)
    np.testing.assert_array_equal(q["counts"], p["counts"])
    sizes = np.diff(q["cu_seqlens"])
    for e in range(El):
        c = int(q["counts"][e])
        assert sizes[e] == (0 if c == 0 else 1 << (c - 1).bit_length())
        seg = q["src_of"][q["cu_seqlens"][e]:q["cu_seqlens"][e + 1]]
        np.testing.assert_array_equal(seg[:c], p["src_of"][p["cu_seqlens"][e]:p["cu_seqlens"][e] + c])
        assert np.all(seg[c:] == -1)
        assert np.all(q["w_perm"][q["cu_seqlens"][e] + c:q["cu_seqlens"][e + 1]] == 0)
    # every routed slot appears exactly once; maps are mutually inverse
    for r, i in enumerate(q["src_of"]):
        if i >= 0:
            assert q["row_of"][i] == r
            np.testing.assert_array_equal(q["x_perm"][r], hid[i // K])
            assert q["w_perm"][r] == w.reshape(-1)[i]
    assert (q["row_of"] >= 0).sum() == q["counts"].sum()


def test_next_pow2():
    assert [oracle.next_pow2(n) for n in [0, 1, 2, 3, 4, 5, 859, 991, 1024, 1025]] == \
        [0, 1, 2, 4, 4, 8, 1024, 1024, 1024, 2048]


# ------------------------------------------------------------------------ ffn

def test_silu_closed_forms():
    ln3 = math.log(3.0)
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4
    np.testing.assert_allclose(silu(np.array([0.0, ln3, -ln3, 50.0, -50.0])),
                               [0.0, 0.75 * ln3, -0.25 * ln3, 50.0, -50.0 * math.exp(-50.0)],
                               rtol=1e-15, atol=1e-300)


def test_expert_ffn_hand_case_pins_gate_up_order():
    # H=2, I=1: gate row picks x0, up row picks x1, w2 = [1, 2]^T
    ln3 = math.log(3.0)
    w13 = np.array([[1.0, 0.0], [0.0, 1.0]])
    w2 = np.array([[1.0], [2.0]])
    y = oracle.expert_ffn(np.array([[ln3, 2.0]]), w13, w2)
    # silu(ln 3) * 2 = 1.5 ln 3; a swapped gate/up would give silu(2) * ln 3
    np.testing.assert_allclose(y[0], [1.5 * ln3, 3.0 * ln3], rtol=1e-15)


def test_grouped_ffn_matches_scalar_loops():
    rng = np.random.default_rng(7)
    T, K, E, H, I = 5, 2, 3, 8, 4
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    hid = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ws = [(f32_to_bf16_bits(rng.standard_normal((2 * I, H)).astype(np.float32)),
           f32_to_bf16_bits(rng.standard_normal((H, I)).astype(np.float32))) for _ in range(E)]
    p = oracle.permute(idx, w, hid, E, 0, pad_pow2=True)
    y = oracle.grouped_ffn(p["x_perm"], p["cu_seqlens"], p["counts"], lambda e: ws[e], p["w_perm"])
    x64 = bf16_bits_to_f32(hid).astype(np.float64)
    for r, i in enumerate(p["src_of"]):
        if i < 0:
            assert np.all(y[r] == 0)
            continue
        t, k = divmod(int(i), K)
        e = int(idx[t, k])
        W13 = bf16_bits_to_f32(ws[e][0]).astype(np.float64)
        W2 = bf16_bits_to_f32(ws[e][1]).astype(np.float64)
        a = []
        for j in range(I):
            g = sum(x64[t, h] * W13[j, h] for h in range(H))
            u = sum(x64[t, h] * W13[I + j, h] for h in range(H))
            a.append(g / (1.0 + math.exp(-g)) * u)
        for h in range(H):
            want = float(w[t, k]) * sum(a[j] * W2[h, j] for j in range(I))
            assert abs(y[r, h] - want) <= 1e-12 * (1 + abs(want))


# -------------------------------------------------------------------- combine

def test_combine_hand_examples():
    for case in _load("combine_order.json")["cases"]:
        n = len(case["rows"])
        H = 1
        rows = np.array([[int(h, 16)] for h in case["rows"]], dtype=np.uint16).reshape(n, H)
        K = max(n, 1)
        row_of = np.array(list(range(n)) + [-1] * (K - n), dtype=np.int32)
        if n == 0:
            rows = np.zeros((1, H), np.uint16)
        shared = None
        if case["shared"] is not None:
            shared = np.array([[int(case["shared"], 16)]], dtype=np.uint16)
        out = oracle.combine(rows, row_of, 1, K, shared)
        assert int(out[0, 0]) == int(case["out"], 16), case


def test_combine_skips_invalid_slots_and_sums_integers_exactly():
    rng = np.random.default_rng(8)
    T, K, H = 20, 4, 16
    vals = rng.integers(-100, 100, size=(T * K, H)).astype(np.float32)
    rows = f32_to_bf16_bits(vals)
    rows_nan = np.concatenate([rows, np.full((1, H), 0x7FC0, np.uint16)])
    row_of = np.arange(T * K, dtype=np.int32)
    drop = rng.random(T * K) < 0.3
    row_of[drop] = -1
    out = oracle.combine(rows_nan, row_of, T, K)
    want = np.zeros((T, H), np.int64)
    for i in range(T * K):
        if row_of[i] >= 0:
            want[i // K] += vals[i].astype(np.int64)
    # integer sums are exact in binary32, so only the final rounding acts
    import torch
    ref = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16)
    np.testing.assert_array_equal(out, ref.view(torch.int16).numpy().view(np.uint16))
