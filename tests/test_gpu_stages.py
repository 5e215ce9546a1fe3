"""Per-stage parity of the HIP kernels (through the C ABI) with the oracle.

Bit-exact: top-k indices, permute counts / cu_seqlens / maps / rows, FP8
fake-quant outputs and scales, combine outputs given identical rows.
Router weights: rtol 1e-6.  Grouped FFN, per expert against the float64
oracle: Frobenius relative error, every row's relative error and every
element (relative to its row's largest reference magnitude) within 2e-2.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_top_route_moe_amd import ops
from oracle.numerics import bf16_bits_to_f32, f32_to_bf16_bits
from tests.gpu_util import (need_gpu, dev_bf16, host_bits, dev, host, rel_err, stacked_weights,
                            check_rows)

pytestmark = pytest.mark.gpu

FFN_TOL = 2e-2
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def setup_module(module):
    need_gpu()
    assert ops.moe_device_check(0) == 0, "not a gfx950 device"


# ---------------------------------------------------------------------- route

def _route_case(logits, k, row_valid=None, renorm=True):
    ref_idx, ref_w = oracle.route(logits, row_valid, k, renorm)
    idx, w = ops.moe_route(dev(logits), k, None if row_valid is None else dev(row_valid), renorm)
    np.testing.assert_array_equal(host(idx), ref_idx)
    np.testing.assert_allclose(host(w), ref_w, rtol=1e-6, atol=0)


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_route_workloads(name):
    cfg = workloads.CONFIGS[name]
    _route_case(workloads.logits(cfg), cfg.K, workloads.row_valid(cfg))


@pytest.mark.parametrize("T,E,K", [(1, 1, 1), (7, 3, 2), (33, 100, 5), (64, 1024, 32), (300, 256, 8), (5, 65, 32)])
def test_route_shapes_and_ties(T, E, K):
    rng = np.random.default_rng(T * 1000 + E + K)
    logits = rng.integers(-3, 4, size=(T, E)).astype(np.float32)    # many ties
    _route_case(logits, K)
    logits2 = rng.standard_normal((T, E)).astype(np.float32)
    _route_case(logits2, K, renorm=False)
    valid = (rng.random(T) > 0.3).astype(np.uint8)
    _route_case(logits2, K, valid)


@pytest.mark.parametrize("E", [64, 128, 256, 1000])
def test_route_signed_zero_ties(E):
    """Rows of mostly +0 and -0 logits (equal in the order: the lower index
    wins) with a few positive and negative ones, spread over every lane group
    of the wave: the argmax kernels (E > 64) and the rank kernel (E = 64)
    pick the oracle's slots."""
    rng = np.random.default_rng(E)
    T, K = 40, 8
    logits = np.where(rng.random((T, E)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    hot = rng.random((T, E)) < 0.03
    logits[hot] = rng.choice([-1.0, 0.5, 1.0], hot.sum()).astype(np.float32)
    _route_case(logits, K)
    _route_case(logits, K, renorm=False)


@pytest.mark.parametrize("E", [8, 64, 256])
def test_route_nan_and_infinite_logits(E):
    """NaN logits rank as -inf (never hiding a real expert, every id in
    range) and equal infinite logits weigh as equals, as the oracle defines:
    rows with scattered NaNs, all-NaN rows, rows with fewer than K finite
    logits and rows with several +inf, through the rank kernel (E <= 64) and
    the argmax kernel (E > 64)."""
    rng = np.random.default_rng(E + 1)
    T, K = 48, 8
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[rng.random((T, E)) < 0.2] = np.nan
    logits[3] = np.nan
    logits[4] = -np.inf
    logits[5, :] = np.nan
    logits[5, [1, 6]] = [0.5, -2.0]                  # two finite logits, K = 8
    logits[6, [0, 3, 7]] = np.inf
    logits[7, [2, 5]] = [-np.inf, np.nan]
    for renorm in (True, False):
        _route_case(logits, K, renorm=renorm)
    idx, _ = ops.moe_route(dev(logits), K)
    assert host(idx).min() >= 0 and host(idx).max() < E


def test_route_rejects_bad_args():
    x = torch.zeros(4, 8, device="cuda")
    with pytest.raises(RuntimeError):
        ops.moe_route(x, 9)


# ----------------------------------------------------------------- fake quant

def _all_finite_bf16_rows(H=128):
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(bits)
    bits = bits[np.isfinite(f)]
    pad = (-len(bits)) % H
    bits = np.concatenate([bits, np.zeros(pad, np.uint16)])
    return bits.reshape(-1, H)


def test_fake_quant_block_exhaustive():
    rows = _all_finite_bf16_rows(128)
    rng = np.random.default_rng(0)
    rows = rows[rng.permutation(len(rows))]          # mix magnitudes across blocks
    rows = np.concatenate([rows, rng.permutation(rows.reshape(-1)).reshape(rows.shape)])
    rows = rows.reshape(-1, 512)                     # 4 blocks per row
    ref, ref_s = oracle.fake_quant_block(rows, 128)
    scales = torch.empty(rows.shape[0], 4, dtype=torch.float32, device="cuda")
    out = ops.moe_fake_quant_rows(dev_bf16(rows), block_scales=scales)
    np.testing.assert_array_equal(host_bits(out), ref)
    np.testing.assert_array_equal(host(scales), ref_s)


@pytest.mark.parametrize("s", [1.0, 2.0 ** -7, 0.0123, 3.7e-3, 1.0 / 448, 0.3, 1e-30, 7e20])
def test_fake_quant_per_tensor_exhaustive(s):
    rows = _all_finite_bf16_rows(128)
    scale = torch.tensor([s], dtype=torch.float32, device="cuda")
    out = ops.moe_fake_quant_rows(dev_bf16(rows), mode=ops.MOE_FQ_PER_TENSOR, scale=scale)
    ref = oracle.fake_quant_per_tensor(rows, np.float32(s))
    np.testing.assert_array_equal(host_bits(out), ref)


def _near_midpoint_scales(n_pairs=20, spread=3, seed=5):
    """Scales s for which some bf16 value x0 has x0 / s within a few float32
    ulps of a halfway point between two E4M3 values (where a quotient
    computed as x * (1/s) could round the other way)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_pairs):
        e, m = int(rng.integers(-5, 8)), int(rng.integers(0, 7))
        mid = (1.0 + (m + 0.5) / 8.0) * 2.0 ** e
        x0 = np.float32(bf16_bits_to_f32(f32_to_bf16_bits(np.float32(rng.uniform(1, 100) * 10.0 ** rng.integers(-3, 3)))))
        s0 = np.float32(np.float64(x0) / mid)
        q = np.float32(x0) / s0                               # IEEE float32 quotient
        assert abs(np.float64(q) - mid) <= 4 * np.spacing(np.float32(mid)), (x0, s0, q, mid)
        for d in range(-spread, spread + 1):
            out.append(np.array([s0]).view(np.uint32)[0] + np.uint32(d + 2 ** 31) - np.uint32(2 ** 31))
    return np.array(out, np.uint32).view(np.float32)


def test_fake_quant_near_rounding_midpoints():
    """Per-tensor scales built so that quotients land within a few ulps of
    E4M3 halfway points, every finite bf16 value each: bit-exact."""
    rows = _all_finite_bf16_rows(128)
    xd = dev_bf16(rows)
    out = torch.empty_like(xd)
    scale = torch.empty(1, dtype=torch.float32, device="cuda")
    for s in _near_midpoint_scales():
        scale.fill_(float(s))
        ops.moe_fake_quant_rows(xd, out, None, ops.MOE_FQ_PER_TENSOR, scale=scale)
        np.testing.assert_array_equal(host_bits(out), oracle.fake_quant_per_tensor(rows, s), err_msg=str(s))


def _fp4_rows(arrange, seed=11):
    """Every finite bfloat16 value once, as rows of 128: shuffled (blocks of
    mixed magnitude) or sorted by magnitude (blocks of similar magnitude,
    every scale exponent in reach)."""
    flat = _all_finite_bf16_rows(128).reshape(-1)
    if arrange == "shuffled":
        flat = np.random.default_rng(seed).permutation(flat)
    else:
        flat = flat[np.argsort(np.abs(bf16_bits_to_f32(flat)), kind="stable")]
    return flat.reshape(-1, 128)


@pytest.mark.parametrize("arrange", ["shuffled", "sorted"])
def test_fake_quant_mxfp4_exhaustive(arrange):
    rows = _fp4_rows(arrange)
    ref, X = oracle.fake_quant_mxfp4(rows)
    scales = torch.empty(rows.shape[0], 4, dtype=torch.float32, device="cuda")
    out = ops.moe_fake_quant_rows(dev_bf16(rows), mode=ops.MOE_FQ_MXFP4, block=32,
                                  block_scales=scales)
    np.testing.assert_array_equal(host_bits(out), ref)
    np.testing.assert_array_equal(host(scales), X.astype(np.float32))


@pytest.mark.parametrize("g", [1.0, 0.0123, 2.0 ** -20, 1e-30, "calibrated"])
@pytest.mark.parametrize("arrange", ["shuffled", "sorted"])
def test_fake_quant_nvfp4_exhaustive(g, arrange):
    rows = _fp4_rows(arrange)
    if g == "calibrated":
        g = oracle.nvfp4_tensor_scale(oracle.calibrate_amax(rows))
    g = np.float32(g)
    ref, b = oracle.fake_quant_nvfp4(rows, g)
    scales = torch.empty(rows.shape[0], 8, dtype=torch.float32, device="cuda")
    out = ops.moe_fake_quant_rows(dev_bf16(rows), mode=ops.MOE_FQ_NVFP4, block=16,
                                  scale=torch.tensor([g], device="cuda"), block_scales=scales)
    np.testing.assert_array_equal(host_bits(out), ref)
    np.testing.assert_array_equal(host(scales), b.astype(np.float32))


def test_fake_quant_fp4_row_skip_and_calibration():
    rng = np.random.default_rng(12)
    x = f32_to_bf16_bits((rng.standard_normal((21, 256)) * 3).astype(np.float32))
    src = np.where(rng.random(21) < 0.3, -1, np.arange(21)).astype(np.int32)
    mask = src >= 0
    ref, X = oracle.fake_quant_mxfp4(x, mask)
    sc = torch.full((21, 8), 99.0, device="cuda")
    out = ops.moe_fake_quant_rows(dev_bf16(x), row_src=dev(src), mode=ops.MOE_FQ_MXFP4, block=32,
                                  block_scales=sc)
    np.testing.assert_array_equal(host_bits(out), ref)
    np.testing.assert_array_equal(host(sc), X.astype(np.float32))
    g = np.float32(0.004)
    ref, b = oracle.fake_quant_nvfp4(x, g, mask)
    xd = dev_bf16(x)                                  # in place: skipped rows untouched
    ops.moe_fake_quant_rows(xd, xd, dev(src), ops.MOE_FQ_NVFP4, 16, torch.tensor([g], device="cuda"))
    np.testing.assert_array_equal(host_bits(xd), ref)
    # NVFP4 without a tensor scale: calibration only
    amax = torch.zeros(1, device="cuda")
    keep = dev_bf16(x)
    ops.moe_fake_quant_rows(keep, keep, dev(src), ops.MOE_FQ_NVFP4, 16, None, None, amax)
    np.testing.assert_array_equal(host_bits(keep), x)
    assert host(amax)[0] == oracle.calibrate_amax(x, mask)


def test_fake_quant_row_skip_inplace_and_amax():
    rng = np.random.default_rng(1)
    x = f32_to_bf16_bits((rng.standard_normal((37, 256)) * 5).astype(np.float32))
    x[3, :128] = 0
    src = np.where(rng.random(37) < 0.3, -1, np.arange(37)).astype(np.int32)
    mask = src >= 0
    # block mode, out of place, skipped rows copied
    ref, ref_s = oracle.fake_quant_block(x, 128, row_mask=mask)
    scales = torch.full((37, 2), 99.0, device="cuda")
    amax = torch.zeros(1, device="cuda")
    out = ops.moe_fake_quant_rows(dev_bf16(x), row_src=dev(src), block_scales=scales, amax_out=amax)
    np.testing.assert_array_equal(host_bits(out), ref)
    np.testing.assert_array_equal(host(scales), ref_s)
    assert host(amax)[0] == oracle.calibrate_amax(x, mask)
    # per-tensor in place: skipped rows untouched
    s = np.float32(0.01)
    xd = dev_bf16(x)
    ops.moe_fake_quant_rows(xd, xd, dev(src), ops.MOE_FQ_PER_TENSOR, scale=torch.tensor([s], device="cuda"))
    np.testing.assert_array_equal(host_bits(xd), oracle.fake_quant_per_tensor(x, s, row_mask=mask))
    # calibration only, running max over two calls
    amax.zero_()
    ops.moe_fake_quant_rows(dev_bf16(x[:10]), None, None, ops.MOE_FQ_PER_TENSOR, amax_out=amax)
    ops.moe_fake_quant_rows(dev_bf16(x[10:]), None, None, ops.MOE_FQ_PER_TENSOR, amax_out=amax)
    assert host(amax)[0] == oracle.calibrate_amax(x)
    sc = ops.moe_scale_from_amax(amax)
    assert host(sc)[0] == np.float32(oracle.calibrate_amax(x) / np.float32(448))
    # the NVFP4 tensor scale, also on the device: the oracle's closed form
    g = ops.moe_scale_from_amax(amax, mode=ops.MOE_FQ_NVFP4)
    assert host(g)[0] == oracle.nvfp4_tensor_scale(oracle.calibrate_amax(x))
    with pytest.raises(RuntimeError):
        ops.moe_scale_from_amax(amax, mode=ops.MOE_FQ_BLOCK)


# -------------------------------------------------------------------- permute

def _permute_case(idx, w, hid, El, begin=0, pow2=False, capacity=None, sample_rows=None,
                  num_experts=None):
    """``num_experts``: the layer's expert count (ids past it are errors);
    by default the end of the local range."""
    T, K = idx.shape
    ref = oracle.permute(idx, w, hid, El, begin, pow2, num_experts=num_experts)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    cap = ops.moe_permute_capacity(T, K, El, pow2) if capacity is None else capacity
    out = ops.alloc_permuted(T, K, hid.shape[1], El, cap, "cuda")
    for t in (out.counts, out.cu_seqlens, out.row_of, out.src_of):
        t.fill_(12345)                               # stale contents must not leak
    out.w_perm.fill_(7.0)
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), El, begin, pow2, cap, out, dev_error=err,
                        num_experts=num_experts)
    assert host(err)[0] == 0
    np.testing.assert_array_equal(host(p.counts), ref["counts"])
    np.testing.assert_array_equal(host(p.cu_seqlens), ref["cu_seqlens"])
    np.testing.assert_array_equal(host(p.row_of), ref["row_of"])
    used = int(ref["cu_seqlens"][-1])
    np.testing.assert_array_equal(host(p.src_of)[:used], ref["src_of"])
    np.testing.assert_array_equal(host(p.w_perm)[:used], ref["w_perm"])
    assert np.all(host(p.src_of)[used:] == -1) and np.all(host(p.w_perm)[used:] == 0)
    valid = np.nonzero(ref["src_of"] >= 0)[0]
    if sample_rows is not None and len(valid) > sample_rows:
        valid = np.sort(np.random.default_rng(0).choice(valid, sample_rows, replace=False))
    got = host_bits(p.x_perm[torch.from_numpy(valid).cuda()]) if len(valid) else np.zeros((0, hid.shape[1]), np.uint16)
    np.testing.assert_array_equal(got, ref["x_perm"][valid])
    return ref


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_permute_workloads(name):
    cfg = workloads.CONFIGS[name]
    idx, w = oracle.route(workloads.logits(cfg), workloads.row_valid(cfg), cfg.K)
    hid = workloads.hidden(cfg)
    ref = _permute_case(idx, w, hid, cfg.E, 0, cfg.pad_pow2,
                        sample_rows=None if cfg.T <= 512 else 4096)
    if name == "prefill":
        assert int(ref["cu_seqlens"][-1]) == 131072


@pytest.mark.parametrize("seed", range(8))
def test_permute_edge_cases(seed):
    rng = np.random.default_rng(seed)
    T = [1, 2, 37, 100, 513, 1025, 3000, 0][seed]
    K = [1, 2, 4, 8, 3, 8, 6, 2][seed]
    E = [1, 3, 32, 64, 7, 256, 1024, 4][seed]
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    if seed == 3:
        idx[:] = 5                                   # one expert gets everything
    if seed == 4:
        idx[:] = -1                                  # all padding
    w = rng.random((T, K)).astype(np.float32)
    hid = rng.integers(0, 2 ** 16, size=(T, 128), dtype=np.uint64).astype(np.uint16)
    for pow2 in (False, True):
        _permute_case(idx, w, hid, E, 0, pow2)
    if E > 2:                                         # an expert-parallel share
        _permute_case(idx, w, hid, E // 2, E // 4, True, num_experts=E)


@pytest.mark.parametrize("T,K,E,H,El,begin", [
    (512, 8, 1024, 128, 1024, 0),      # 4096 slots: the single-launch path at its limit
    (513, 8, 64, 128, 64, 0),          # 4104 slots: the multi-launch path
    (4096, 1, 5, 128, 5, 0),           # one slot per token
    (500, 8, 2000, 128, 1000, 500),    # an expert-parallel share of 1000 experts
    (100, 8, 2048, 128, 1024, 1024),   # the upper half of 2048 experts (1024 is the limit)
    (3, 2, 4, 8320, 4, 0),             # rows wider than the single launch's up-front loads
    (4096, 8, 1024, 128, 1024, 0),     # 32 chunks per scan thread: its register path at the limit
    (4300, 8, 1024, 128, 1024, 0),     # 34 chunks per scan thread: its loop path
    (4200, 8, 128, 128, 128, 0),       # 33 chunks over 8 scan threads: a short and an empty block
    (4096, 8, 256, 128, 256, 0),       # 32 chunks x 256 experts: the column-read scatter at its limits
    (4097, 8, 256, 128, 256, 0),       # 33 chunks: the scan kernel again
    (2100, 8, 257, 128, 257, 0),       # 17 chunks x 257 experts: the scan kernel
    (2100, 8, 300, 128, 256, 44),      # 17 chunks, an expert-parallel share: the column read
    (3000, 6, 64, 128, 64, 0),         # 96 slots per workgroup: some span two chunks
])
def test_permute_launch_path_boundaries(T, K, E, H, El, begin):
    """Either side of the single-launch permute's limits (4096 slots, 4 row
    vectors per thread loaded up front), at the 1024-local-expert limit,
    either side of the scan kernel's 32 chunks per thread held in registers,
    and either side of the scatter that reads the chunk table's columns
    itself (at most 32 chunks and 256 local experts), including workgroups
    whose slots span two chunks: bit-exact."""
    rng = np.random.default_rng(T * K + E)
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    hid = rng.integers(0, 2 ** 16, size=(T, H), dtype=np.uint64).astype(np.uint16)
    for pow2 in (False, True):
        _permute_case(idx, w, hid, El, begin, pow2, num_experts=E)


@pytest.mark.parametrize("T,K,E,H,pow2,begin_el", [
    (64, 2, 8, 256, False, None),        # one launch
    (300, 8, 16, 512, True, (4, 8)),     # one launch, pow2 buckets, an expert-parallel share
    (700, 8, 32, 384, False, None),      # 5600 slots: the multi-launch path
    (3, 2, 4, 8320, True, None),         # rows wider than the one launch's up-front loads
    (2100, 8, 64, 256, True, None),      # 17 chunks: the scatter that reads the table's columns
    (5000, 8, 300, 128, False, None),    # 40 chunks, 300 experts: the scan kernel
])
def test_permute_dispatch_fp8_equals_quantize_then_permute(T, K, E, H, pow2, begin_el):
    """MOE_PERMUTE_DISPATCH_FP8: the permuted rows are the 1x128 FP8 dispatch
    fake-quant of the token rows (the oracle's block quantizer, then its
    permute), bit for bit; rows include all-zero blocks, negative zeros,
    subnormals and large magnitudes."""
    rng = np.random.default_rng(T + H)
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    vals = rng.standard_normal((T, H)).astype(np.float32) * rng.choice([1e-3, 1.0, 1e4], (T, 1))
    hid = f32_to_bf16_bits(vals.astype(np.float32))
    hid[0, :128] = 0                                 # an all-zero block
    hid[0, 128:136] = 0x8000                         # negative zeros
    hid[-1, :16] = np.arange(1, 17, dtype=np.uint16)  # subnormals
    begin, El = begin_el if begin_el else (0, E)
    hq, _ = oracle.fake_quant_block(hid, 128)
    ref = oracle.permute(idx, w, hq, El, begin, pow2)
    cap = ops.moe_permute_capacity(T, K, El, pow2)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), El, begin, pow2, cap, dev_error=err,
                        dispatch_fp8=True, num_experts=E)
    assert host(err)[0] == 0
    np.testing.assert_array_equal(host(p.row_of), ref["row_of"])
    rows = np.nonzero(ref["src_of"] >= 0)[0]
    np.testing.assert_array_equal(host_bits(p.x_perm)[rows], ref["x_perm"][rows])


def test_empty_batch_every_stage():
    """T = 0 through route, permute, both FFN modes and combine: no error,
    empty outputs, all-zero counts and cu_seqlens."""
    E, K, H, I = 8, 2, 256, 128
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx, w = ops.moe_route(torch.zeros(0, E, device="cuda"), K)
    assert tuple(idx.shape) == (0, K) and tuple(w.shape) == (0, K)
    hid = torch.zeros(0, H, dtype=torch.bfloat16, device="cuda")
    for pow2 in (False, True):
        p = ops.moe_permute(idx, w, hid, E, 0, pow2, dev_error=err)
        np.testing.assert_array_equal(host(p.counts), np.zeros(E, np.int32))
        np.testing.assert_array_equal(host(p.cu_seqlens), np.zeros(E + 1, np.int32))
        assert p.x_perm.shape[0] == 0
    w13 = torch.zeros(E, 2 * I, H, dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros(E, H, I, dtype=torch.bfloat16, device="cuda")
    y = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13, w2, p.w_perm, dev_error=err)
    assert tuple(y.shape) == (0, H)
    w13p, w2p = ops.moe_pack_ffn_weights(w13, w2)
    y = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13p, w2p, p.w_perm, dev_error=err,
                            flags=ops.MOE_FFN_ALL | ops.MOE_FFN_PACKED_WEIGHTS)
    assert tuple(y.shape) == (0, H)
    out = ops.moe_combine(y, p.row_of, 0, K, dev_error=err)
    assert tuple(out.shape) == (0, H)
    torch.cuda.synchronize()
    assert host(err)[0] == 0


@pytest.mark.parametrize("T,K,E,El,begin", [
    (64, 2, 8, 8, 0),          # one launch
    (300, 8, 64, 32, 16),      # one launch, an expert-parallel share
    (700, 8, 64, 64, 0),       # the multi-launch path, scan fused into the scatter
    (4096, 8, 256, 256, 0),    # the multi-launch path, the scatter reading the table's columns
    (5000, 8, 300, 300, 0),    # the multi-launch path with the scan kernel
])
def test_permute_expert_id_out_of_range_fails_closed(T, K, E, El, begin):
    """Router ids at or past the layer's expert count raise
    MOE_DEVERR_EXPERT_RANGE and are not routed; every map and row still
    matches the oracle (which drops them the same way); ids of other ranks'
    experts and negative ids of any value are not errors."""
    rng = np.random.default_rng(T + E)
    idx = rng.integers(-3, E, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    hid = rng.integers(0, 2 ** 16, size=(T, 128), dtype=np.uint64).astype(np.uint16)
    for bad in (False, True):
        if bad:
            idx[rng.integers(0, T, 3), rng.integers(0, K, 3)] = [E, E + 7, 2 ** 30]
        ref = oracle.permute(idx, w, hid, El, begin, False, num_experts=E)
        assert ref["expert_range_error"] == bad
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), El, begin, False, dev_error=err,
                            num_experts=E)
        torch.cuda.synchronize()
        assert host(err)[0] == (ops.MOE_DEVERR_EXPERT_RANGE if bad else 0)
        for key in ("counts", "cu_seqlens", "row_of"):
            np.testing.assert_array_equal(host(getattr(p, key)), ref[key])
        used = int(ref["cu_seqlens"][-1])
        np.testing.assert_array_equal(host(p.src_of)[:used], ref["src_of"])
        rows = np.nonzero(ref["src_of"] >= 0)[0]
        np.testing.assert_array_equal(host_bits(p.x_perm)[rows], ref["x_perm"][rows])
    with pytest.raises(RuntimeError):                 # a share past the layer's experts
        ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), El, E - El + 1, num_experts=E)


@pytest.mark.parametrize("T,K,E,cap", [
    (64, 4, 8, 100),          # the single-launch path; 256 rows are needed
    (2100, 8, 64, 10000),     # the scatter that reads the chunk table's columns; 16800 needed
    (5000, 8, 300, 20000),    # the scan kernel; 40000 needed
])
def test_permute_capacity_overflow_is_flagged_not_written(T, K, E, cap):
    rng = np.random.default_rng(9)
    H = 128
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    hid = rng.integers(0, 2 ** 16, size=(T, H), dtype=np.uint64).astype(np.uint16)
    guard = 16
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = ops.alloc_permuted(T, K, H, E, cap + guard, "cuda")
    out.x_perm.fill_(0)
    out.src_of.fill_(-7)
    ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), E, 0, False, cap, out, dev_error=err)
    assert host(err)[0] == ops.MOE_DEVERR_CAPACITY
    assert np.all(host(out.src_of)[cap:] == -7)       # nothing written past capacity
    assert np.all(host_bits(out.x_perm[cap:]) == 0)
    ro = host(out.row_of)
    assert ro.max() < cap


# -------------------------------------------------------------------- combine

def _combine_case(rows, row_of, T, K, shared=None, scale=None):
    rows_q = rows
    if scale is not None:
        mask = np.zeros(len(rows), bool)
        mask[row_of[row_of >= 0]] = True
        rows_q = oracle.fake_quant_per_tensor(rows, np.float32(scale), row_mask=mask)
    ref = oracle.combine(rows_q, row_of, T, K, shared)
    out = ops.moe_combine(dev_bf16(rows), dev(row_of), T, K,
                          None if shared is None else dev_bf16(shared),
                          None if scale is None else torch.tensor([scale], dtype=torch.float32, device="cuda"))
    np.testing.assert_array_equal(host_bits(out), ref)


def test_combine_golden_cases():
    with open(os.path.join(GOLDEN, "combine_order.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        n = len(case["rows"])
        H = 128
        K = max(n, 1)
        rows = np.zeros((K, H), np.uint16)
        for i, h in enumerate(case["rows"]):
            rows[i, :] = int(h, 16)
        row_of = np.array(list(range(n)) + [-1] * (K - n), np.int32)
        shared = None if case["shared"] is None else np.full((1, H), int(case["shared"], 16), np.uint16)
        out = ops.moe_combine(dev_bf16(rows), dev(row_of), 1, K, None if shared is None else dev_bf16(shared))
        assert np.all(host_bits(out) == int(case["out"], 16)), case["what"]


@pytest.mark.parametrize("T,K,H", [(1, 1, 128), (50, 8, 256), (512, 8, 2048), (37, 3, 7168)])
def test_combine_random_rows(T, K, H):
    rng = np.random.default_rng(T + K + H)
    R = T * K + 5
    vals = rng.standard_normal((R, H)).astype(np.float32) * rng.choice([1e-3, 1.0, 1e3], (R, 1)).astype(np.float32)
    rows = f32_to_bf16_bits(vals)
    rows[0, :16] = np.arange(1, 17, dtype=np.uint16)          # subnormals
    rows[1, :16] = np.arange(0x8001, 0x8011, dtype=np.uint16)
    perm = rng.permutation(R)[: T * K].astype(np.int32)
    row_of = np.where(rng.random(T * K) < 0.2, -1, perm).astype(np.int32)
    shared = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    _combine_case(rows, row_of, T, K)
    _combine_case(rows, row_of, T, K, shared)
    # fused QDQ: a typical scale, an arbitrary one, and one outside the
    # reciprocal's exact range (the kernel then divides)
    for s in (3.0 / 448, 0.0123, 1e-30):
        _combine_case(rows, row_of, T, K, shared, scale=float(np.float32(s)))
    # slot-major [K, T, H] layout: row_of[t*K + k] = k*T + t
    t_idx, k_idx = np.divmod(np.arange(T * K), K)
    _combine_case(rows, (k_idx * T + t_idx).astype(np.int32), T, K, shared)


@pytest.mark.parametrize("scale", [3.0 / 448, 0.0123, 1e-30])
def test_combine_qdq_table_form(scale):
    """Combines of at least 2^20 16-byte vectors take the table form of the
    FP8 QDQ (each workgroup tabulates the quantizer over the 32768
    magnitudes, the sign is copied).  Every bf16 bit pattern as a routed row:
    the table form bit-identical to the arithmetic form that smaller combines
    take, for every pattern (NaNs and infinities too), and both bit-exact
    against the oracle for the finite ones; then random K=2 rows with a
    shared slot at table-form size against the oracle."""
    s = float(np.float32(scale))
    sc = torch.tensor([s], dtype=torch.float32, device="cuda")
    T, H = 2048, 4096                     # T * H / 8 = 2^20 vectors
    pat = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rows = np.tile(pat, T * H // 65536).reshape(T, H)
    row_of = np.arange(T, dtype=np.int32)
    big = host_bits(ops.moe_combine(dev_bf16(rows), dev(row_of), T, 1, None, sc))
    small = host_bits(ops.moe_combine(dev_bf16(rows[:16]), dev(row_of[:16]), 16, 1, None, sc))
    np.testing.assert_array_equal(big[:16], small)
    np.testing.assert_array_equal(big[16:32], small)
    finite = ((pat & 0x7F80) != 0x7F80).reshape(16, H)
    fin_rows = np.where(finite, rows[:16], 0).astype(np.uint16)   # the oracle takes finite values
    ref = oracle.combine(oracle.fake_quant_per_tensor(fin_rows, np.float32(s)), row_of[:16], 16, 1)
    np.testing.assert_array_equal(small[finite], ref[finite])
    rng = np.random.default_rng(21)
    K = 2
    R = T * K + 3
    vals = rng.standard_normal((R, H)).astype(np.float32) * rng.choice([1e-3, 1.0, 1e3], (R, 1)).astype(np.float32)
    perm = rng.permutation(R)[: T * K].astype(np.int32)
    row_of = np.where(rng.random(T * K) < 0.2, -1, perm).astype(np.int32)
    shared = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    _combine_case(f32_to_bf16_bits(vals), row_of, T, K, shared, scale=s)


def _check_case(seed=7, T=37, K=4, H=256):
    rng = np.random.default_rng(seed)
    rows = f32_to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32))
    row_of = rng.permutation(T * K).astype(np.int32)
    row_of[rng.random(T * K) < 0.2] = -1
    shared = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    return rows, row_of, shared


def _run_check(rows, row_of, T, K, out, shared, state=None):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.moe_combine_check(dev_bf16(rows), dev(row_of), T, K, dev_bf16(out), dev_bf16(shared),
                          state, err)
    torch.cuda.synchronize()
    return int(err.item())


def test_combine_check_layout():
    """Page 1's layout check: rows that re-sum (in the combine order) to the
    fused kernel's output pass and mark the buffer checked; any difference
    raises MOE_DEVERR_LAYOUT; a checked buffer is not checked again; a
    padding-only batch defers the check; without a state word every call
    checks.  Expected outputs are the oracle's combine."""
    T, K, H = 37, 4, 256
    rows, row_of, shared = _check_case(T=T, K=K, H=H)
    want = oracle.combine(rows, row_of, T, K, shared)
    bad = want.copy()
    bad[5, 17] ^= 1                                   # one bit of one element
    # the same buffer read with another layout (every row one position on)
    other = np.where(row_of >= 0, (row_of + 1) % (T * K), -1).astype(np.int32)
    assert not np.array_equal(oracle.combine(rows, other, T, K, shared), want)
    state = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert _run_check(rows, row_of, T, K, want, shared, state) == 0
    assert int(state.item()) == 1
    assert _run_check(rows, row_of, T, K, bad, shared, state) == 0      # checked once
    assert int(state.item()) == 1
    state.zero_()
    assert _run_check(rows, row_of, T, K, bad, shared, state) == ops.MOE_DEVERR_LAYOUT
    assert int(state.item()) == 0
    assert _run_check(rows, other, T, K, want, shared, state) == ops.MOE_DEVERR_LAYOUT
    assert int(state.item()) == 0
    # padding-only batch (every slot -1): consistent output, but nothing routed
    pad = np.full(T * K, -1, np.int32)
    assert _run_check(rows, pad, T, K, oracle.combine(rows, pad, T, K, shared), shared, state) == 0
    assert int(state.item()) == 0
    # no state: every call checks
    assert _run_check(rows, row_of, T, K, want, shared) == 0
    assert _run_check(rows, row_of, T, K, bad, shared) == ops.MOE_DEVERR_LAYOUT


@pytest.mark.parametrize("wrong", [False, True])
def test_combine_check_in_graph_after_padding_warmup(wrong):
    """A graph captured before any routed batch holds the check: the replay
    over a padding-only batch defers it, the first replay with routed rows
    performs it (raising on a changed layout), later replays skip it."""
    T, K, H = 29, 3, 128
    rows, row_of, shared = _check_case(seed=8, T=T, K=K, H=H)
    want = oracle.combine(rows, row_of, T, K, shared)
    layout = np.where(row_of >= 0, (row_of + 1) % (T * K), -1).astype(np.int32) if wrong else row_of
    d_rows, d_shared = dev_bf16(rows), dev_bf16(shared)
    d_row_of = torch.full((T * K,), -1, dtype=torch.int32, device="cuda")   # padding warmup
    d_out = dev_bf16(oracle.combine(rows, np.full(T * K, -1, np.int32), T, K, shared))
    state = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ops.moe_combine_check(d_rows, d_row_of, T, K, d_out, d_shared, state, err)
    g.replay()
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and int(state.item()) == 0          # deferred
    d_row_of.copy_(dev(layout))
    d_out.copy_(dev_bf16(want))
    g.replay()
    torch.cuda.synchronize()
    if wrong:
        assert int(err.item()) == ops.MOE_DEVERR_LAYOUT and int(state.item()) == 0
    else:
        assert int(err.item()) == 0 and int(state.item()) == 1
        d_out.view(torch.int16)[0, 0] += 1                           # later corruption
        g.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0 and int(state.item()) == 1      # checked once


def test_combine_row_out_of_range_flagged():
    rows = np.zeros((4, 128), np.uint16)
    row_of = np.array([0, 9, 1, -1], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.moe_combine(dev_bf16(rows), dev(row_of), 2, 2, dev_error=err)
    assert host(err)[0] == ops.MOE_DEVERR_ROW_RANGE


# ---------------------------------------------------------------- grouped FFN

def _ffn_case(cfg, idx, w, hid, host_w, w13, w2, pow2=False, experts=None, tol=FFN_TOL):
    ref = oracle.permute(idx, w, hid, cfg.E, 0, pow2)
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), cfg.E, 0, pow2)
    y = torch.zeros(p.x_perm.shape, dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13, w2, p.w_perm, y, dev_error=err)
    assert host(err)[0] == 0
    cu, cnt = ref["cu_seqlens"], ref["counts"]
    experts = range(cfg.E) if experts is None else experts
    worst = 0.0
    for e in experts:
        n = int(cnt[e])
        if n == 0:
            continue
        r0 = int(cu[e])
        x = oracle.bf16_bits_to_f64(ref["x_perm"][r0:r0 + n])
        want = oracle.expert_ffn(x, *host_w[e]) * ref["w_perm"][r0:r0 + n, None].astype(np.float64)
        got = bf16_bits_to_f32(host_bits(y[r0:r0 + n]))
        st = check_rows(got, want, tol, what=f"expert {e} ({n} rows)")
        worst = max(worst, st["worst_row"])
        seg_end = int(cu[e + 1])
        if seg_end > r0 + n:                          # pow2 padding rows are never written
            assert np.all(host_bits(y[r0 + n:seg_end]) == 0)
    return worst


@pytest.mark.parametrize("m,skew", [(1, 1.0), (37, 1.0), (100, 8.0), (512, 8.0), (512, 1.0)])
def test_ffn_page_shapes(m, skew):
    """The MoonEP test's shapes: m tokens, top-4 of 32 experts, router skew."""
    cfg = workloads.MoEConfig("t", 9, T=m, H=256, E=32, K=4, I=128, hot_experts=8 if skew > 1 else 0)
    lg = workloads.logits(cfg)
    idx, w = oracle.route(lg, None, 4)
    hid = workloads.hidden(cfg)
    w13, w2, host_w = stacked_weights(cfg)
    _ffn_case(cfg, idx, w, hid, host_w, w13, w2)
    _ffn_case(cfg, idx, w, hid, host_w, w13, w2, pow2=True)


@pytest.mark.parametrize("name", ["tiny", "balanced", "skewed"])
def test_ffn_workloads(name):
    cfg = workloads.CONFIGS[name]
    idx, w = oracle.route(workloads.logits(cfg), None, cfg.K)
    hid = workloads.hidden(cfg)
    w13, w2, host_w = stacked_weights(cfg)
    worst = _ffn_case(cfg, idx, w, hid, host_w, w13, w2)
    print(f"{name}: worst row rel err {worst:.3e}")


def test_ffn_one_big_segment_many_tiles():
    """One expert with 1000 rows: 8 m-tiles, ragged tail."""
    cfg = workloads.MoEConfig("t", 11, T=1000, H=512, E=4, K=1, I=256)
    idx = np.full((1000, 1), 2, np.int32)
    w = np.ones((1000, 1), np.float32)
    hid = workloads.hidden(cfg)
    w13, w2, host_w = stacked_weights(cfg)
    _ffn_case(cfg, idx, w, hid, host_w, w13, w2)


def test_ffn_stage_split_equals_all():
    cfg = workloads.MoEConfig("t", 12, T=200, H=256, E=8, K=2, I=256)
    idx, w = oracle.route(workloads.logits(cfg), None, 2)
    hid = workloads.hidden(cfg)
    w13, w2, _ = stacked_weights(cfg)
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), cfg.E)
    ws = torch.empty(ops.moe_grouped_ffn_workspace_bytes(p.x_perm.shape[0], 8, 256, 256), dtype=torch.uint8, device="cuda")
    y1 = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13, w2, p.w_perm)
    y2 = torch.empty_like(y1)
    ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13, w2, p.w_perm, y2, ops.MOE_FFN_GATE_UP, ws)
    ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13, w2, p.w_perm, y2, ops.MOE_FFN_DOWN, ws)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_ffn_deterministic():
    cfg = workloads.CONFIGS["tiny"]
    idx, w = oracle.route(workloads.logits(cfg), None, cfg.K)
    w13, w2, _ = stacked_weights(cfg)
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(workloads.hidden(cfg)), cfg.E)
    a = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13, w2, p.w_perm)
    b = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13, w2, p.w_perm)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("H,I,T", [(512, 256, 300), (128, 128, 40), (384, 256, 700),
                                   (256, 256, 2000), (384, 256, 1700), (128, 384, 1600)])
def test_ffn_packed_weights(H, I, T):
    """Packed weights in MFMA fragment order: the packing is the documented
    permutation of the input, and the fragment-streaming GEMM matches the
    oracle.  The cases cover both workgroup widths (4 waves when segments
    average under 128 rows, 8 above), a partial column block (H/64 or 2I/64
    not a multiple of the column tiles per workgroup) and several m-tiles
    per expert with ragged tails."""
    cfg = workloads.MoEConfig("t", 13, T=T, H=H, E=6, K=2, I=I, hot_experts=2)
    idx, w = oracle.route(workloads.logits(cfg), None, 2)
    hid = workloads.hidden(cfg)
    w13, w2, host_w = stacked_weights(cfg)
    w13p, w2p = ops.moe_pack_ffn_weights(w13, w2)
    G = cfg.E
    # w2 [G, H, I]: K-step ks, column tile ct = rows 64ct.., fragment f =
    # rows +16f.., lane l -> row + l%16, cols 32ks + 8(l/16) .. +8
    got = host_bits(w2p).reshape(G, I // 32, H // 64, 4, 4, 16, 8)     # g ks ct f (l/16) (l%16) 8
    want = host_bits(w2).reshape(G, H // 64, 4, 16, I // 32, 4, 8).transpose(0, 4, 1, 2, 5, 3, 6)
    np.testing.assert_array_equal(got, want)
    # w13: column tile ct = gate rows 32ct.. (fragments 0, 1) then up rows
    g13 = host_bits(w13p).reshape(G, H // 32, I // 32, 4, 4, 16, 8)
    w13h = host_bits(w13)
    gate = w13h[:, :I].reshape(G, I // 32, 2, 16, H // 32, 4, 8).transpose(0, 4, 1, 2, 5, 3, 6)
    up = w13h[:, I:].reshape(G, I // 32, 2, 16, H // 32, 4, 8).transpose(0, 4, 1, 2, 5, 3, 6)
    np.testing.assert_array_equal(g13[:, :, :, :2], gate)
    np.testing.assert_array_equal(g13[:, :, :, 2:], up)
    # the GEMM on packed weights against the oracle
    ref = oracle.permute(idx, w, hid, G, 0, False)
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), G)
    y = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13p, w2p, p.w_perm,
                            flags=ops.MOE_FFN_ALL | ops.MOE_FFN_PACKED_WEIGHTS)
    for e in range(G):
        n, r0 = int(ref["counts"][e]), int(ref["cu_seqlens"][e])
        if n == 0:
            continue
        x = oracle.bf16_bits_to_f64(ref["x_perm"][r0:r0 + n])
        want_y = oracle.expert_ffn(x, *host_w[e]) * ref["w_perm"][r0:r0 + n, None].astype(np.float64)
        check_rows(bf16_bits_to_f32(host_bits(y[r0:r0 + n])), want_y, FFN_TOL, what=f"expert {e}")
    # and it agrees closely with the row-major kernel (different summation order)
    y2 = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13, w2, p.w_perm)
    used = int(ref["cu_seqlens"][-1])
    assert rel_err(bf16_bits_to_f32(host_bits(y[:used])), bf16_bits_to_f32(host_bits(y2[:used]))) < 1e-2


@pytest.mark.parametrize("fp8", [False, True])
def test_ffn_tall_tiles_streamed_across_tiles(fp8):
    """The tall tiles run persistently, each workgroup taking several tiles
    in turn, with the next tile's weights and activation chunks fetched
    during the current tile's last steps and its epilogue.  Enough tiles for
    about three per workgroup, tile to tile changes of segment length (a
    single row, 16 and 17 rows, full 256-row tiles, experts spanning two
    tall tiles, empty experts between), every expert against the oracle per
    row and element; with BF16 weights and with FP8 weights (against the
    oracle on the dequantized weights)."""
    rng = np.random.default_rng(11)
    G, H, I = 200, 1024, 512
    sizes = rng.integers(90, 220, G)
    sizes[:14] = [0, 1, 16, 17, 255, 256, 257, 300, 511, 512, 128, 129, 0, 2]
    sizes = [int(n) for n in rng.permutation(sizes)]
    assert 96 <= sum(sizes) // G < 256
    cfg = workloads.MoEConfig("t", 43, T=sum(sizes), H=H, E=G, K=1, I=I)
    idx = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(sizes)])[:, None]
    idx = rng.permutation(idx)
    w = rng.uniform(0.5, 1.5, idx.shape).astype(np.float32)
    hid = workloads.hidden(cfg)
    w13, w2, host_w = stacked_weights(cfg)
    ref = oracle.permute(idx, w, hid, G, 0, False)
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), G)
    if fp8:
        q13, s13, q2, s2 = ops.moe_pack_ffn_weights_fp8(w13, w2)
        y = ops.moe_grouped_ffn_fp8(p.x_perm, p.cu_seqlens, p.counts, q13, s13, q2, s2, p.w_perm)
    else:
        w13p, w2p = ops.moe_pack_ffn_weights(w13, w2)
        y = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13p, w2p, p.w_perm,
                                flags=ops.MOE_FFN_ALL | ops.MOE_FFN_PACKED_WEIGHTS)
    torch.cuda.synchronize()
    got = bf16_bits_to_f32(host_bits(y))
    for e in range(G):
        n, r0 = int(ref["counts"][e]), int(ref["cu_seqlens"][e])
        if n == 0:
            continue
        x = oracle.bf16_bits_to_f64(ref["x_perm"][r0:r0 + n])
        rs = ref["w_perm"][r0:r0 + n, None].astype(np.float64)
        wts = [oracle.quantize_weight_blocks(m)[2] for m in host_w[e]] if fp8 else host_w[e]
        check_rows(got[r0:r0 + n], oracle.expert_ffn(x, *wts) * rs, FFN_TOL,
                   what=f"expert {e} ({n} rows)")


@pytest.mark.parametrize("fp8", [False, True])
def test_ffn_tall_tiles_streamed_at_the_limits(fp8):
    """The streamed tall kernel at its limits: 1024 groups (its LDS tile
    table full) and H = I = 128, so each K loop has two chunks and the next
    tile's first chunk goes out with the current tile's first one; many
    tiles per workgroup, empty groups among them; BF16 and FP8 weights."""
    rng = np.random.default_rng(12)
    G, H, I = 1024, 128, 128
    sizes = [int(n) for n in rng.integers(90, 230, G)]
    for e in rng.choice(G, 40, replace=False):
        sizes[e] = 0
    sizes[3], sizes[500] = 257, 1
    assert 96 <= sum(sizes) // G < 256
    cfg = workloads.MoEConfig("t", 44, T=sum(sizes), H=H, E=G, K=1, I=I)
    idx = rng.permutation(np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(sizes)])[:, None])
    w = rng.uniform(0.5, 1.5, idx.shape).astype(np.float32)
    hid = workloads.hidden(cfg)
    w13, w2, host_w = stacked_weights(cfg)
    ref = oracle.permute(idx, w, hid, G, 0, False)
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), G)
    if fp8:
        q13, s13, q2, s2 = ops.moe_pack_ffn_weights_fp8(w13, w2)
        y = ops.moe_grouped_ffn_fp8(p.x_perm, p.cu_seqlens, p.counts, q13, s13, q2, s2, p.w_perm)
    else:
        w13p, w2p = ops.moe_pack_ffn_weights(w13, w2)
        y = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13p, w2p, p.w_perm,
                                flags=ops.MOE_FFN_ALL | ops.MOE_FFN_PACKED_WEIGHTS)
    torch.cuda.synchronize()
    got = bf16_bits_to_f32(host_bits(y))
    for e in range(G):
        n, r0 = int(ref["counts"][e]), int(ref["cu_seqlens"][e])
        if n == 0:
            continue
        x = oracle.bf16_bits_to_f64(ref["x_perm"][r0:r0 + n])
        rs = ref["w_perm"][r0:r0 + n, None].astype(np.float64)
        wts = [oracle.quantize_weight_blocks(m)[2] for m in host_w[e]] if fp8 else host_w[e]
        check_rows(got[r0:r0 + n], oracle.expert_ffn(x, *wts) * rs, FFN_TOL,
                   what=f"expert {e} ({n} rows)")


def test_ffn_tall_tiles_edges():
    """Segments averaging 96..255 rows take the tall tiles (256 rows per
    workgroup, half a column tile per wave): segments of exactly 128, 129,
    255, 256 and 257 rows (the last spills into a second tall tile), a
    single row, an empty expert, and a down projection whose wave tiles do
    not fill the last workgroup (H / 32 = 12 of 16); every expert against
    the oracle per row and element, with BF16 and with FP8 weights."""
    sizes = [128, 129, 255, 256, 257, 1, 0]
    G, H, I = len(sizes), 384, 256
    cfg = workloads.MoEConfig("t", 41, T=sum(sizes), H=H, E=G, K=1, I=I)
    assert 96 <= sum(sizes) // G < 256
    idx = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(sizes)])[:, None]
    idx = np.random.default_rng(3).permutation(idx)
    w = np.random.default_rng(4).uniform(0.5, 1.5, idx.shape).astype(np.float32)
    hid = workloads.hidden(cfg)
    w13, w2, host_w = stacked_weights(cfg)
    ref = oracle.permute(idx, w, hid, G, 0, False)
    p = ops.moe_permute(dev(idx), dev(w), dev_bf16(hid), G)
    w13p, w2p = ops.moe_pack_ffn_weights(w13, w2)
    y = ops.moe_grouped_ffn(p.x_perm, p.cu_seqlens, p.counts, w13p, w2p, p.w_perm,
                            flags=ops.MOE_FFN_ALL | ops.MOE_FFN_PACKED_WEIGHTS)
    q13, s13, q2, s2 = ops.moe_pack_ffn_weights_fp8(w13, w2)
    y8 = ops.moe_grouped_ffn_fp8(p.x_perm, p.cu_seqlens, p.counts, q13, s13, q2, s2, p.w_perm)
    torch.cuda.synchronize()
    for e in range(G):
        n, r0 = int(ref["counts"][e]), int(ref["cu_seqlens"][e])
        if n == 0:
            continue
        x = oracle.bf16_bits_to_f64(ref["x_perm"][r0:r0 + n])
        rs = ref["w_perm"][r0:r0 + n, None].astype(np.float64)
        check_rows(bf16_bits_to_f32(host_bits(y[r0:r0 + n])),
                   oracle.expert_ffn(x, *host_w[e]) * rs, FFN_TOL, what=f"bf16 expert {e} ({n} rows)")
        deq = [oracle.quantize_weight_blocks(m)[2] for m in host_w[e]]
        check_rows(bf16_bits_to_f32(host_bits(y8[r0:r0 + n])),
                   oracle.expert_ffn(x, *deq) * rs, FFN_TOL, what=f"fp8w expert {e} ({n} rows)")



@pytest.mark.parametrize("pattern", ["overlap", "huge"])
@pytest.mark.parametrize("path,capacity", [("bf16", 300), ("bf16", 600), ("fp8w", 300),
                                           ("fp8w", 600), ("w8a8", 300)])
def test_ffn_segments_past_the_workspace_fail_closed(path, capacity, pattern):
    """Segments that each lie inside [0, capacity) but overlap (every group
    starting at row 0), or counts far above the capacity, would place the
    later groups' m-tiles of the intermediate past the workspace's
    ceil(capacity / 128) + G m-tiles.  Every fragment-order kernel (the
    128-row tiles at a mean under 96 rows per group, the streamed tall tiles
    at 96..255, FP8 weights, FP8 rows) reports ROW_RANGE for them and
    writes nothing past the workspace or the output."""
    G, H, I = 4, 256, 256
    cfg = workloads.MoEConfig("t", 45, T=capacity, H=H, E=G, K=1, I=I)
    w13, w2, _ = stacked_weights(cfg)
    x = dev_bf16(workloads.hidden(cfg))
    if pattern == "overlap":
        counts = np.full(G, capacity, np.int32)
        seg = np.zeros(G + 1, np.int32)
    else:
        counts = np.array([2**31 - 1, 100, 2**31 - 1, 50], np.int32)
        seg = np.array([0, 0, 0, 100, capacity], np.int32)
    seg[G] = capacity
    d_counts, d_seg = dev(counts), dev(seg)
    y_all = torch.full((capacity + 8, H), 1.5, dtype=torch.bfloat16, device="cuda")
    y = y_all[:capacity]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if path == "w8a8":
        need = ops.moe_grouped_ffn_w8a8_workspace_bytes(capacity, G, H, I)
    else:
        need = ops.moe_grouped_ffn_workspace_bytes(capacity, G, H, I)
    ws = torch.zeros(need + 4096, dtype=torch.uint8, device="cuda")
    ws[need:] = 0xA5
    if path == "bf16":
        w13p, w2p = ops.moe_pack_ffn_weights(w13, w2)
        ops.moe_grouped_ffn(x, d_seg, d_counts, w13p, w2p, None, y,
                            ops.MOE_FFN_ALL | ops.MOE_FFN_PACKED_WEIGHTS, ws[:need], err)
    elif path == "fp8w":
        q13, s13, q2, s2 = ops.moe_pack_ffn_weights_fp8(w13, w2)
        ops.moe_grouped_ffn_fp8(x, d_seg, d_counts, q13, s13, q2, s2, None, y,
                                workspace=ws[:need], dev_error=err)
    else:
        q13, s13, q2, s2 = ops.moe_pack_ffn_weights_fp8(w13, w2, k128=True)
        xq, xs = ops.moe_quant_rows_fp8(x)
        ops.moe_grouped_ffn_w8a8(xq, xs, d_seg, d_counts, q13, s13, q2, s2, None, y,
                                 workspace=ws[:need], dev_error=err)
    torch.cuda.synchronize()
    assert host(err)[0] == ops.MOE_DEVERR_ROW_RANGE
    assert bool((ws[need:] == 0xA5).all())
    assert bool((y_all[capacity:] == 1.5).all())


@pytest.mark.parametrize("nvec", [1, 255, 1024, 4097, 300001])
def test_copy_bytes(nvec):
    """The streaming copy behind the copy-bandwidth figure: exact, including
    sizes that end part-way through a workgroup's run of 4 x 256 vectors."""
    src = torch.randint(-2**31, 2**31 - 1, (nvec * 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros(nvec * 4 + 4, dtype=torch.int32, device="cuda")
    ops.moe_copy_bytes(src, dst[:nvec * 4])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nvec * 4], src)
    assert int(dst[nvec * 4:].abs().sum()) == 0   # nothing written past the end


def test_read_bytes():
    """The read-only stream behind the read-bandwidth figure: it reads its
    whole input (a ragged size included) without error and writes nothing
    to the sink unless a thread's checksum equals the marker, which these
    inputs never produce."""
    sink = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    for nvec in (1, 2047, 300001):
        src = torch.zeros(nvec * 4, dtype=torch.int32, device="cuda")
        ops.moe_read_bytes(src, sink)
    torch.cuda.synchronize()
    assert int(sink.sum()) == 0
