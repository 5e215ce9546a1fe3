"""Python binding of the C ABI: one function per entry point, same names.

Argument marshalling only.  torch supplies device memory and the current
stream; every step of the path runs in the HIP kernels of ``libmoe.so``.
Outputs that the caller does not pass are allocated here with
``torch.empty`` on the input's device.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from ._lib import load, check

MOE_ROUTE_RENORM = 1
MOE_PERMUTE_PAD_POW2 = 1
MOE_PERMUTE_DISPATCH_FP8 = 2
MOE_FFN_GATE_UP, MOE_FFN_DOWN, MOE_FFN_ALL, MOE_FFN_PACKED_WEIGHTS = 1, 2, 3, 4
MOE_FQ_PER_TENSOR, MOE_FQ_BLOCK, MOE_FQ_NVFP4, MOE_FQ_MXFP4 = 0, 1, 2, 3
MOE_DEVERR_ROW_RANGE, MOE_DEVERR_CAPACITY, MOE_DEVERR_LAYOUT, MOE_DEVERR_EXPERT_RANGE = 1, 2, 3, 4
MOE_ERR_SCRATCH = -6
MOE_FP8_LAYOUT_K128 = 1


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _want(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def moe_device_check(device: int = 0) -> int:
    return load().moe_device_check(device)


def moe_route(logits: torch.Tensor, k: int, row_valid: Optional[torch.Tensor] = None,
              renormalize: bool = True, topk_idx=None, topk_w=None, stream=None):
    _want(logits, torch.float32, "logits")
    T, E = logits.shape
    dev = logits.device
    if row_valid is not None:
        _want(row_valid, torch.uint8, "row_valid")
    topk_idx = torch.empty(T, k, dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    topk_w = torch.empty(T, k, dtype=torch.float32, device=dev) if topk_w is None else topk_w
    check("moe_route", load().moe_route(
        _ptr(logits), _ptr(row_valid), T, E, k, MOE_ROUTE_RENORM if renormalize else 0,
        _ptr(topk_idx), _ptr(topk_w), _stream(stream)))
    return topk_idx, topk_w


def moe_permute_capacity(T: int, K: int, num_local_experts: int, pad_pow2: bool = False) -> int:
    return load().moe_permute_capacity(T, K, num_local_experts, MOE_PERMUTE_PAD_POW2 if pad_pow2 else 0)


def moe_permute_workspace_bytes(T: int, K: int, num_local_experts: int, pad_pow2: bool = False) -> int:
    return load().moe_permute_workspace_bytes(T, K, num_local_experts,
                                              MOE_PERMUTE_PAD_POW2 if pad_pow2 else 0)


@dataclass
class Permuted:
    counts: torch.Tensor
    cu_seqlens: torch.Tensor
    x_perm: torch.Tensor
    row_of: torch.Tensor
    src_of: torch.Tensor
    w_perm: torch.Tensor


def alloc_permuted(T: int, K: int, H: int, num_local_experts: int, capacity: int,
                   device) -> Permuted:
    i32 = dict(dtype=torch.int32, device=device)
    return Permuted(
        counts=torch.empty(num_local_experts, **i32),
        cu_seqlens=torch.empty(num_local_experts + 1, **i32),
        x_perm=torch.empty(capacity, H, dtype=torch.bfloat16, device=device),
        row_of=torch.empty(T * K, **i32),
        src_of=torch.empty(capacity, **i32),
        w_perm=torch.empty(capacity, dtype=torch.float32, device=device),
    )


def moe_permute(topk_idx: torch.Tensor, topk_w: torch.Tensor, hidden: torch.Tensor,
                num_local_experts: int, expert_begin: int = 0, pad_pow2: bool = False,
                capacity: Optional[int] = None, out: Optional[Permuted] = None,
                workspace: Optional[torch.Tensor] = None,
                dev_error: Optional[torch.Tensor] = None, stream=None,
                dispatch_fp8: bool = False, num_experts: Optional[int] = None) -> Permuted:
    """``dispatch_fp8``: the rows are written FP8 fake-quantized in 1 x 128
    blocks (MOE_PERMUTE_DISPATCH_FP8).  ``num_experts``: the layer's total
    expert count (ids at or past it raise MOE_DEVERR_EXPERT_RANGE); by
    default the end of the local range, i.e. all experts local."""
    _want(topk_idx, torch.int32, "topk_idx")
    _want(topk_w, torch.float32, "topk_w")
    _want(hidden, torch.bfloat16, "hidden")
    T, K = topk_idx.shape
    H = hidden.shape[1]
    flags = (MOE_PERMUTE_PAD_POW2 if pad_pow2 else 0) | (MOE_PERMUTE_DISPATCH_FP8 if dispatch_fp8 else 0)
    if num_experts is None:
        num_experts = expert_begin + num_local_experts
    lib = load()
    if capacity is None:
        capacity = out.x_perm.shape[0] if out is not None else lib.moe_permute_capacity(
            T, K, num_local_experts, flags)
    if out is None:
        out = alloc_permuted(T, K, H, num_local_experts, capacity, hidden.device)
    ws_need = lib.moe_permute_workspace_bytes(T, K, num_local_experts, flags)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=hidden.device)
    check("moe_permute", lib.moe_permute(
        _ptr(topk_idx), _ptr(topk_w), _ptr(hidden), T, K, H, num_experts, expert_begin,
        num_local_experts,
        flags, capacity, _ptr(out.counts), _ptr(out.cu_seqlens), _ptr(out.x_perm),
        _ptr(out.row_of), _ptr(out.src_of), _ptr(out.w_perm), _ptr(workspace),
        workspace.numel(), _ptr(dev_error), _stream(stream)))
    return out


def moe_permute_noalloc_scratch_bytes() -> int:
    return load().moe_permute_noalloc_scratch_bytes()


def moe_permute_noalloc(topk_idx: torch.Tensor, topk_w: torch.Tensor, hidden: torch.Tensor,
                        num_local_experts: int, out: Permuted, expert_begin: int = 0,
                        pad_pow2: bool = False, dev_error: Optional[torch.Tensor] = None,
                        stream=None, dispatch_fp8: bool = False,
                        num_experts: Optional[int] = None) -> Permuted:
    """``moe_permute`` with the library's fixed device scratch instead of a
    workspace: the caller passes the output buffers (``out``, whose
    ``x_perm`` rows are the capacity); nothing is allocated here either."""
    _want(topk_idx, torch.int32, "topk_idx")
    _want(topk_w, torch.float32, "topk_w")
    _want(hidden, torch.bfloat16, "hidden")
    T, K = topk_idx.shape
    H = hidden.shape[1]
    flags = (MOE_PERMUTE_PAD_POW2 if pad_pow2 else 0) | (MOE_PERMUTE_DISPATCH_FP8 if dispatch_fp8 else 0)
    if num_experts is None:
        num_experts = expert_begin + num_local_experts
    check("moe_permute_noalloc", load().moe_permute_noalloc(
        _ptr(topk_idx), _ptr(topk_w), _ptr(hidden), T, K, H, num_experts, expert_begin,
        num_local_experts, flags, out.x_perm.shape[0], _ptr(out.counts), _ptr(out.cu_seqlens),
        _ptr(out.x_perm), _ptr(out.row_of), _ptr(out.src_of), _ptr(out.w_perm), _ptr(dev_error),
        _stream(stream)))
    return out


def moe_grouped_ffn_workspace_bytes(capacity: int, num_groups: int, H: int, I: int) -> int:
    return load().moe_grouped_ffn_workspace_bytes(capacity, num_groups, H, I)


def moe_grouped_ffn(x: torch.Tensor, cu_seqlens: torch.Tensor, counts: torch.Tensor,
                    w13: torch.Tensor, w2: torch.Tensor, row_scale: Optional[torch.Tensor] = None,
                    y: Optional[torch.Tensor] = None, flags: int = MOE_FFN_ALL,
                    workspace: Optional[torch.Tensor] = None,
                    dev_error: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _want(x, torch.bfloat16, "x")
    _want(w13, torch.bfloat16, "w13")
    _want(w2, torch.bfloat16, "w2")
    _want(cu_seqlens, torch.int32, "cu_seqlens")
    _want(counts, torch.int32, "counts")
    if row_scale is not None:
        _want(row_scale, torch.float32, "row_scale")
    capacity, H = x.shape
    G, two_i, H2 = w13.shape
    I = two_i // 2
    if H2 != H or tuple(w2.shape) != (G, H, I):
        raise ValueError("weight shapes do not match x")
    if counts.numel() != G or cu_seqlens.numel() != G + 1:
        raise ValueError("counts / cu_seqlens do not match the number of groups")
    lib = load()
    y = torch.empty(capacity, H, dtype=torch.bfloat16, device=x.device) if y is None else y
    need = lib.moe_grouped_ffn_workspace_bytes(capacity, G, H, I)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    check("moe_grouped_ffn", lib.moe_grouped_ffn(
        _ptr(x), _ptr(cu_seqlens), _ptr(counts), G, H, I, _ptr(w13), _ptr(w2), _ptr(row_scale),
        _ptr(y), capacity, flags, _ptr(workspace), workspace.numel(), _ptr(dev_error),
        _stream(stream)))
    return y


def moe_pack_ffn_weights(w13: Optional[torch.Tensor], w2: Optional[torch.Tensor],
                         w13_packed: Optional[torch.Tensor] = None,
                         w2_packed: Optional[torch.Tensor] = None, stream=None):
    """Copy w13 [G,2I,H] / w2 [G,H,I] into the grouped GEMM's packed layout."""
    if w13 is not None:
        _want(w13, torch.bfloat16, "w13")
        G, two_i, H = w13.shape
        I = two_i // 2
    else:
        _want(w2, torch.bfloat16, "w2")
        G, H, I = w2.shape
    if w13 is not None and w13_packed is None:
        w13_packed = torch.empty_like(w13)
    if w2 is not None and w2_packed is None:
        w2_packed = torch.empty_like(w2)
    check("moe_pack_ffn_weights", load().moe_pack_ffn_weights(
        _ptr(w13), _ptr(w2), G, H, I, _ptr(w13_packed), _ptr(w2_packed),
        _stream(stream)))
    return w13_packed, w2_packed


def moe_grouped_ffn_fp8(x: torch.Tensor, cu_seqlens: torch.Tensor, counts: torch.Tensor,
                        w13q: torch.Tensor, w13_scales: torch.Tensor, w2q: torch.Tensor,
                        w2_scales: torch.Tensor, row_scale: Optional[torch.Tensor] = None,
                        y: Optional[torch.Tensor] = None, flags: int = MOE_FFN_ALL,
                        workspace: Optional[torch.Tensor] = None,
                        dev_error: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The grouped FFN with FP8 weights from moe_pack_ffn_weights_fp8 (codes
    uint8 [G,2I,H] / [G,H,I] in packed order, tile scales float32)."""
    _want(x, torch.bfloat16, "x")
    _want(w13q, torch.uint8, "w13q")
    _want(w2q, torch.uint8, "w2q")
    _want(w13_scales, torch.float32, "w13_scales")
    _want(w2_scales, torch.float32, "w2_scales")
    _want(cu_seqlens, torch.int32, "cu_seqlens")
    _want(counts, torch.int32, "counts")
    if row_scale is not None:
        _want(row_scale, torch.float32, "row_scale")
    capacity, H = x.shape
    G, two_i, H2 = w13q.shape
    I = two_i // 2
    if H2 != H or tuple(w2q.shape) != (G, H, I):
        raise ValueError("weight shapes do not match x")
    if (tuple(w13_scales.shape) != (G, two_i // 128, H // 128)
            or tuple(w2_scales.shape) != (G, H // 128, I // 128)):
        raise ValueError("scale shapes do not match the weights")
    if counts.numel() != G or cu_seqlens.numel() != G + 1:
        raise ValueError("counts / cu_seqlens do not match the number of groups")
    lib = load()
    y = torch.empty(capacity, H, dtype=torch.bfloat16, device=x.device) if y is None else y
    need = lib.moe_grouped_ffn_workspace_bytes(capacity, G, H, I)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    check("moe_grouped_ffn_fp8", lib.moe_grouped_ffn_fp8(
        _ptr(x), _ptr(cu_seqlens), _ptr(counts), G, H, I, _ptr(w13q), _ptr(w13_scales),
        _ptr(w2q), _ptr(w2_scales), _ptr(row_scale), _ptr(y), capacity, flags, _ptr(workspace),
        workspace.numel(), _ptr(dev_error), _stream(stream)))
    return y


def moe_pack_ffn_weights_fp8(w13: Optional[torch.Tensor], w2: Optional[torch.Tensor],
                             k128: bool = False, stream=None):
    """Quantize w13 [G,2I,H] / w2 [G,H,I] to E4M3 with one float32 scale per
    128 x 128 tile, codes in the packed order of moe_grouped_ffn_fp8 (or,
    with ``k128``, of moe_grouped_ffn_w8a8).  Returns
    ``(w13q, w13_scales, w2q, w2_scales)`` (None for an absent input)."""
    if w13 is not None:
        _want(w13, torch.bfloat16, "w13")
        G, two_i, H = w13.shape
        I = two_i // 2
    else:
        _want(w2, torch.bfloat16, "w2")
        G, H, I = w2.shape
    dev = (w13 if w13 is not None else w2).device
    w13q = w13s = w2q = w2s = None
    if w13 is not None:
        w13q = torch.empty(G, 2 * I, H, dtype=torch.uint8, device=dev)
        w13s = torch.empty(G, 2 * I // 128, H // 128, dtype=torch.float32, device=dev)
    if w2 is not None:
        w2q = torch.empty(G, H, I, dtype=torch.uint8, device=dev)
        w2s = torch.empty(G, H // 128, I // 128, dtype=torch.float32, device=dev)
    check("moe_pack_ffn_weights_fp8", load().moe_pack_ffn_weights_fp8(
        _ptr(w13), _ptr(w2), G, H, I, _ptr(w13q), _ptr(w13s), _ptr(w2q), _ptr(w2s),
        MOE_FP8_LAYOUT_K128 if k128 else 0, _stream(stream)))
    return w13q, w13s, w2q, w2s


def moe_quant_rows_fp8(inp: torch.Tensor, row_src: Optional[torch.Tensor] = None,
                       codes: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None, stream=None):
    """bf16 rows [R, H] -> E4M3 codes uint8 [R, H] and float32 scales
    [H/128, stride] (K-block-major, stride = scales.shape[1] >= R)."""
    _want(inp, torch.bfloat16, "inp")
    R, H = inp.shape
    if codes is None:
        codes = torch.empty(R, H, dtype=torch.uint8, device=inp.device)
    if scales is None:
        scales = torch.empty(H // 128, max(R, 1), dtype=torch.float32, device=inp.device)
    _want(codes, torch.uint8, "codes")
    _want(scales, torch.float32, "scales")
    if row_src is not None:
        _want(row_src, torch.int32, "row_src")
    check("moe_quant_rows_fp8", load().moe_quant_rows_fp8(
        _ptr(inp), R, H, _ptr(row_src), _ptr(codes), _ptr(scales), scales.shape[1],
        _stream(stream)))
    return codes, scales


def moe_grouped_ffn_w8a8_workspace_bytes(capacity: int, num_groups: int, H: int, I: int) -> int:
    return load().moe_grouped_ffn_w8a8_workspace_bytes(capacity, num_groups, H, I)


def moe_grouped_ffn_w8a8(xq: torch.Tensor, x_scales: torch.Tensor, cu_seqlens: torch.Tensor,
                         counts: torch.Tensor, w13q: torch.Tensor, w13_scales: torch.Tensor,
                         w2q: torch.Tensor, w2_scales: torch.Tensor,
                         row_scale: Optional[torch.Tensor] = None,
                         y: Optional[torch.Tensor] = None, flags: int = MOE_FFN_ALL,
                         workspace: Optional[torch.Tensor] = None,
                         dev_error: Optional[torch.Tensor] = None, stream=None,
                         scale_src: Optional[torch.Tensor] = None, scale_div: int = 1) -> torch.Tensor:
    """The grouped FFN on FP8 rows (moe_quant_rows_fp8) and FP8 weights
    (moe_pack_ffn_weights_fp8 with ``k128=True``) on the FP8 matrix cores.
    ``scale_src`` / ``scale_div``: row r's scales are those of row
    ``scale_src[r] // scale_div`` of ``x_scales`` (the permute's src_of and K)."""
    _want(xq, torch.uint8, "xq")
    _want(x_scales, torch.float32, "x_scales")
    _want(w13q, torch.uint8, "w13q")
    _want(w2q, torch.uint8, "w2q")
    _want(w13_scales, torch.float32, "w13_scales")
    _want(w2_scales, torch.float32, "w2_scales")
    _want(cu_seqlens, torch.int32, "cu_seqlens")
    _want(counts, torch.int32, "counts")
    if row_scale is not None:
        _want(row_scale, torch.float32, "row_scale")
    capacity, H = xq.shape
    G, two_i, H2 = w13q.shape
    I = two_i // 2
    if H2 != H or tuple(w2q.shape) != (G, H, I):
        raise ValueError("weight shapes do not match xq")
    if x_scales.shape[0] != H // 128 or (scale_src is None and x_scales.shape[1] < capacity):
        raise ValueError("x_scales must be [H/128, >= capacity] (or >= T with scale_src)")
    if scale_src is not None:
        _want(scale_src, torch.int32, "scale_src")
    if counts.numel() != G or cu_seqlens.numel() != G + 1:
        raise ValueError("counts / cu_seqlens do not match the number of groups")
    lib = load()
    y = torch.empty(capacity, H, dtype=torch.bfloat16, device=xq.device) if y is None else y
    need = lib.moe_grouped_ffn_w8a8_workspace_bytes(capacity, G, H, I)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xq.device)
    check("moe_grouped_ffn_w8a8", lib.moe_grouped_ffn_w8a8(
        _ptr(xq), _ptr(x_scales), x_scales.shape[1], _ptr(scale_src), scale_div, _ptr(cu_seqlens),
        _ptr(counts), G, H, I,
        _ptr(w13q), _ptr(w13_scales), _ptr(w2q), _ptr(w2_scales), _ptr(row_scale), _ptr(y),
        capacity, flags, _ptr(workspace), workspace.numel(), _ptr(dev_error), _stream(stream)))
    return y


def moe_fake_quant_rows(inp: torch.Tensor, out: Optional[torch.Tensor] = None,
                        row_src: Optional[torch.Tensor] = None, mode: int = MOE_FQ_BLOCK,
                        block: int = 128, scale: Optional[torch.Tensor] = None,
                        block_scales: Optional[torch.Tensor] = None,
                        amax_out: Optional[torch.Tensor] = None, stream=None):
    _want(inp, torch.bfloat16, "in")
    n_rows, H = inp.shape
    if out is None and (mode in (MOE_FQ_BLOCK, MOE_FQ_MXFP4) or scale is not None):
        out = torch.empty_like(inp)
    if row_src is not None:
        _want(row_src, torch.int32, "row_src")
    check("moe_fake_quant_rows", load().moe_fake_quant_rows(
        _ptr(inp), _ptr(out), n_rows, H, _ptr(row_src), mode, block, _ptr(scale),
        _ptr(block_scales), _ptr(amax_out), _stream(stream)))
    return out


def moe_scale_from_amax(amax: torch.Tensor, scale: Optional[torch.Tensor] = None,
                        stream=None, mode: int = MOE_FQ_PER_TENSOR) -> torch.Tensor:
    """``mode``: MOE_FQ_PER_TENSOR (FP8 scale) or MOE_FQ_NVFP4 (tensor scale)."""
    _want(amax, torch.float32, "amax")
    scale = torch.empty(1, dtype=torch.float32, device=amax.device) if scale is None else scale
    check("moe_scale_from_amax", load().moe_scale_from_amax(_ptr(amax), _ptr(scale), mode,
                                                            _stream(stream)))
    return scale


def moe_combine(rows: torch.Tensor, row_of: torch.Tensor, T: int, K: int,
                shared: Optional[torch.Tensor] = None, qdq_scale: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, dev_error: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    _want(rows, torch.bfloat16, "rows")
    _want(row_of, torch.int32, "row_of")
    num_rows, H = rows.shape
    out = torch.empty(T, H, dtype=torch.bfloat16, device=rows.device) if out is None else out
    check("moe_combine", load().moe_combine(
        _ptr(rows), num_rows, _ptr(row_of), _ptr(shared), T, K, H, _ptr(qdq_scale), _ptr(out),
        _ptr(dev_error), _stream(stream)))
    return out


def moe_combine_check(rows: torch.Tensor, row_of: torch.Tensor, T: int, K: int,
                      kernel_out: torch.Tensor, shared: Optional[torch.Tensor] = None,
                      state: Optional[torch.Tensor] = None,
                      dev_error: Optional[torch.Tensor] = None, stream=None) -> None:
    """Check that ``rows`` re-summed in the combine order reproduce
    ``kernel_out`` bit for bit (MOE_DEVERR_LAYOUT into dev_error otherwise);
    ``state`` is an optional zero-initialised int32 device word that makes the
    check happen once per buffer, on its first batch with routed rows."""
    _want(rows, torch.bfloat16, "rows")
    _want(row_of, torch.int32, "row_of")
    _want(kernel_out, torch.bfloat16, "kernel_out")
    if state is not None:
        _want(state, torch.int32, "state")
    num_rows, H = rows.shape
    check("moe_combine_check", load().moe_combine_check(
        _ptr(rows), num_rows, _ptr(row_of), _ptr(shared), T, K, H, _ptr(kernel_out), _ptr(state),
        _ptr(dev_error), _stream(stream)))


def moe_read_bytes(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    n = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < 65536:
        raise ValueError("sink must hold at least 64 KiB")
    check("moe_read_bytes", load().moe_read_bytes(_ptr(src), n, _ptr(sink), _stream(stream)))


def moe_copy_bytes(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    check("moe_copy_bytes", load().moe_copy_bytes(_ptr(src), _ptr(dst), n, _stream(stream)))
