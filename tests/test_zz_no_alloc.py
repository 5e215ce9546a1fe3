"""moe_permute_noalloc (the permute on the library's fixed device scratch,
for callers that cannot allocate) against moe_permute with a caller
workspace: every output bit for bit, on two calls in a row (the second with
a smaller input, so stale scratch contents from the first must not leak),
both through the multi-launch paths that use the scratch; an input past the
scratch is refused before anything is enqueued."""

import numpy as np
import pytest
import torch

from combine_top_route_moe_amd import ops
from tests.gpu_util import need_gpu, dev, dev_bf16, host, host_bits

pytestmark = pytest.mark.gpu


def setup_module(module):
    need_gpu()


def _inputs(T, K, E, H, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    hid = rng.integers(0, 2 ** 16, size=(T, H), dtype=np.uint64).astype(np.uint16)
    return dev(idx), dev(w), dev_bf16(hid)


def _same(a: ops.Permuted, b: ops.Permuted):
    for key in ("counts", "cu_seqlens", "row_of", "src_of", "w_perm"):
        np.testing.assert_array_equal(host(getattr(a, key)), host(getattr(b, key)), err_msg=key)
    used = int(host(a.cu_seqlens)[-1])
    src = host(a.src_of)[:used]
    rows = torch.from_numpy(np.nonzero(src >= 0)[0]).cuda()
    np.testing.assert_array_equal(host_bits(a.x_perm[rows]), host_bits(b.x_perm[rows]))


@pytest.mark.parametrize("pow2,fp8", [(False, False), (True, True)])
def test_noalloc_permute_matches_workspace_permute(pow2, fp8):
    assert ops.moe_permute_noalloc_scratch_bytes() == 4 << 20
    # first a batch with the one-workgroup scan kernel (32 chunks), then a
    # smaller one whose scan is fused into the scatter (6 chunks)
    for (T, K, E, H, seed) in ((4096, 8, 256, 256, 1), (700, 8, 64, 128, 2)):
        idx, w, hid = _inputs(T, K, E, H, seed)
        cap = ops.moe_permute_capacity(T, K, E, pow2)
        err_a = torch.zeros(1, dtype=torch.int32, device="cuda")
        err_b = torch.zeros(1, dtype=torch.int32, device="cuda")
        a = ops.moe_permute(idx, w, hid, E, 0, pow2, cap, dev_error=err_a, dispatch_fp8=fp8)
        b = ops.alloc_permuted(T, K, H, E, cap, "cuda")
        for t in (b.counts, b.cu_seqlens, b.row_of, b.src_of):
            t.fill_(-9)
        ops.moe_permute_noalloc(idx, w, hid, E, b, 0, pow2, dev_error=err_b, dispatch_fp8=fp8)
        torch.cuda.synchronize()
        assert int(err_a.item()) == 0 and int(err_b.item()) == 0
        _same(a, b)


def test_noalloc_permute_refuses_inputs_past_its_scratch():
    # 1 048 576 slots need 4 MiB of ranks plus the chunk table: more than the scratch
    T, K, E, H = 131072, 8, 128, 128
    need = ops.moe_permute_workspace_bytes(T, K, E)
    assert need > ops.moe_permute_noalloc_scratch_bytes()
    idx = torch.zeros(T, K, dtype=torch.int32, device="cuda")
    w = torch.zeros(T, K, dtype=torch.float32, device="cuda")
    hid = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    out = ops.alloc_permuted(T, K, H, E, T * K, "cuda")
    with pytest.raises(RuntimeError) as info:
        ops.moe_permute_noalloc(idx, w, hid, E, out)
    assert info.value.status == ops.MOE_ERR_SCRATCH
