"""One MoE layer on one GPU: buffers owned once, the ABI calls in order.

Order of the stages (titles of the pages they come from):
  route           "[Kernel] DeepEP dispatch-combine kernel integration"
  dispatch QDQ    "Add MoE dispatch/combine fake quantization for vLLM's
                  DeepGEMM Mega-MoE", "How it works"
  permute         "[Distributed][MoonEP] BF16 integration of MoonEP balanced
                  EP backend", "Purpose"; "[Bugfix][MoE] Size the permute
                  scratch from its inputs"
  grouped FFN     MoonEP page, commit message adding the modular experts
  shared expert   Mega-MoE page: a fused shared expert's slot, added last
  combine (+QDQ)  Mega-MoE page, PR summary and "How it works"

Every buffer is allocated once in the constructor (torch is the allocator);
``forward`` only enqueues kernels on the current stream, never synchronizes
and never allocates, so it can be timed back to back or captured in a graph.
"""

from __future__ import annotations

from typing import Callable, Dict, List, Optional, Tuple

import torch

from . import ops


_FP4 = {"nvfp4": (ops.MOE_FQ_NVFP4, 16), "mxfp4": (ops.MOE_FQ_MXFP4, 32)}


class MoELayer:
    def __init__(self, T: int, H: int, E: int, K: int, I: int, device="cuda",
                 shared_I: int = 0, dispatch_block: int = 0, combine_qdq: bool = False,
                 pad_pow2: bool = False, renormalize: bool = True, expert_begin: int = 0,
                 num_local_experts: Optional[int] = None, dispatch_fp4: Optional[str] = None,
                 combine_fp4: Optional[str] = None):
        """``dispatch_block`` (128) selects the FP8 dispatch quantizer (run
        inside the permute as it copies the rows: the same bits as quantizing
        first) and
        ``combine_qdq`` the FP8 combine quantizer; ``dispatch_fp4`` /
        ``combine_fp4`` ("nvfp4" or "mxfp4") the FP4 ones instead.  NVFP4
        tensor scales live in ``dispatch_scale`` / ``combine_scale`` (device
        scalars the caller fills, or ``calibrate_combine_scale``)."""
        for fmt in (dispatch_fp4, combine_fp4):
            if fmt not in (None, "nvfp4", "mxfp4"):
                raise ValueError(f"unknown FP4 format {fmt!r}")
        self.T, self.H, self.E, self.K, self.I = T, H, E, K, I
        self.dispatch_fp4, self.combine_fp4 = dispatch_fp4, combine_fp4
        self.shared_I = shared_I
        self.dispatch_block = dispatch_block
        self.combine_qdq = combine_qdq
        self.pad_pow2 = pad_pow2
        self.renormalize = renormalize
        self.expert_begin = expert_begin
        self.El = E if num_local_experts is None else num_local_experts
        dev = torch.device(device)
        self.device = dev
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        bf = dict(dtype=torch.bfloat16, device=dev)

        self.topk_idx = torch.empty(T, K, **i32)
        self.topk_w = torch.empty(T, K, **f32)
        # the FP8 dispatch quantizer in 1 x 128 blocks runs inside the permute
        # (MOE_PERMUTE_DISPATCH_FP8); the other quantizers write hidden_q first
        self.fuse_dispatch = dispatch_block == 128 and not dispatch_fp4
        self.hidden_q = (torch.empty(T, H, **bf)
                         if (dispatch_block or dispatch_fp4) and not self.fuse_dispatch else None)
        self.dispatch_scale = torch.zeros(1, **f32) if dispatch_fp4 == "nvfp4" else None
        self.capacity = ops.moe_permute_capacity(T, K, self.El, pad_pow2)
        self.perm = ops.alloc_permuted(T, K, H, self.El, self.capacity, dev)
        self.perm_ws = torch.empty(max(ops.moe_permute_workspace_bytes(T, K, self.El, pad_pow2), 1),
                                   dtype=torch.uint8, device=dev)
        self.ffn_ws = torch.empty(max(ops.moe_grouped_ffn_workspace_bytes(self.capacity, self.El, H, I), 1),
                                  dtype=torch.uint8, device=dev)
        self.y_perm = torch.empty(self.capacity, H, **bf)
        self.out = torch.empty(T, H, **bf)
        self.dev_error = torch.zeros(1, **i32)
        self.combine_scale = (torch.zeros(1, **f32) if combine_qdq or combine_fp4 == "nvfp4"
                              else None)
        self.amax = torch.zeros(1, **f32)
        if shared_I:
            # the shared expert depends only on `hidden`: forward() runs it on
            # a side stream, concurrently with the routed path (default
            # priority), and joins it before the combine
            self.side = torch.cuda.Stream(device=dev)
            self.shared_out = torch.empty(T, H, **bf)
            self.shared_cu = torch.tensor([0, T], **i32)
            self.shared_counts = torch.tensor([T], **i32)
            self.shared_ws = torch.empty(max(ops.moe_grouped_ffn_workspace_bytes(T, 1, H, shared_I), 1),
                                         dtype=torch.uint8, device=dev)
        else:
            self.shared_out = None
        self.w13 = self.w2 = self.shared_w13 = self.shared_w2 = None
        self.packed = False
        self.fp8_weights = False
        self.w8a8 = False

    # ------------------------------------------------------------------ weights
    def set_weights(self, w13: torch.Tensor, w2: torch.Tensor,
                    shared_w13: Optional[torch.Tensor] = None,
                    shared_w2: Optional[torch.Tensor] = None, pack: bool = True,
                    fp8=False) -> None:
        """Device bf16 weights: w13 [E_l, 2I, H], w2 [E_l, H, I] (local experts);
        the shared expert's [2Is, H] and [H, Is] (run as a single group).

        With ``pack`` (the default) the weights are copied once into the
        grouped GEMM's packed layout (``moe_pack_ffn_weights``) and the
        row-major tensors are not referenced afterwards.  With ``fp8`` they
        are quantized once instead to E4M3 codes with 128 x 128 tile scales
        (``moe_pack_ffn_weights_fp8``), routed and shared experts alike, and
        the FFN stages read those (``moe_grouped_ffn_fp8``).  With
        ``fp8="w8a8"`` the activations are FP8 too: the dispatch rows are
        quantized for real (``moe_quant_rows_fp8``, 1 x 128 blocks) before the
        permute, which moves their codes, and both GEMMs run on the FP8
        matrix cores (``moe_grouped_ffn_w8a8``); this replaces the dispatch
        fake-quant.  Requires H % 256 == 0."""
        if shared_w13 is not None and shared_w13.dim() == 2:
            shared_w13, shared_w2 = shared_w13.unsqueeze(0), shared_w2.unsqueeze(0)
        if fp8 not in (False, True, "w8a8"):
            raise ValueError(f"unknown fp8 mode {fp8!r}")
        self.w8a8 = fp8 == "w8a8"
        self.fp8_weights = bool(fp8)
        if self.w8a8:
            self._setup_w8a8()
            q13, s13, q2, s2 = ops.moe_pack_ffn_weights_fp8(w13, w2, k128=True)
            self.w13, self.w2 = (q13, s13), (q2, s2)
            self.shared_w13 = self.shared_w2 = None
            if shared_w13 is not None:
                q13, s13, q2, s2 = ops.moe_pack_ffn_weights_fp8(shared_w13, shared_w2, k128=True)
                self.shared_w13, self.shared_w2 = (q13, s13), (q2, s2)
            self.packed = True
            return
        if fp8:
            self.packed = True
            q13, s13, q2, s2 = ops.moe_pack_ffn_weights_fp8(w13, w2)
            self.w13, self.w2 = (q13, s13), (q2, s2)
            self.shared_w13 = self.shared_w2 = None
            if shared_w13 is not None:
                q13, s13, q2, s2 = ops.moe_pack_ffn_weights_fp8(shared_w13, shared_w2)
                self.shared_w13, self.shared_w2 = (q13, s13), (q2, s2)
            return
        self.packed = pack
        if pack:
            w13, w2 = ops.moe_pack_ffn_weights(w13, w2)
            if shared_w13 is not None:
                shared_w13, shared_w2 = ops.moe_pack_ffn_weights(shared_w13, shared_w2)
        self.w13, self.w2 = w13, w2
        self.shared_w13, self.shared_w2 = shared_w13, shared_w2

    def _setup_w8a8(self) -> None:
        """Buffers of the FP8 path: the [T, H] rows' codes and scales, the
        permuted codes (moved by the permute as 2-byte units), workspaces."""
        T, H, K, dev = self.T, self.H, self.K, self.device
        if H % 256:
            raise ValueError("the FP8 path needs H % 256 == 0 (codes move as 2-byte units)")
        if self.dispatch_fp4:
            raise ValueError("the FP8 path quantizes the dispatch rows itself (no FP4 dispatch)")
        self.hq = torch.empty(T, H, dtype=torch.uint8, device=dev)
        self.hs = torch.empty(H // 128, max(T, 1), dtype=torch.float32, device=dev)
        # the permutation moves the codes: x_perm holds [cap, H] bytes as
        # [cap, H/2] 2-byte units (the maps are those of any permute)
        self.perm = ops.alloc_permuted(T, K, H // 2, self.El, self.capacity, dev)
        self.ffn_ws = torch.empty(
            max(ops.moe_grouped_ffn_w8a8_workspace_bytes(self.capacity, self.El, H, self.I), 1),
            dtype=torch.uint8, device=dev)
        if self.shared_I:
            self.shared_ws = torch.empty(
                max(ops.moe_grouped_ffn_w8a8_workspace_bytes(T, 1, H, self.shared_I), 1),
                dtype=torch.uint8, device=dev)

    def _ffn(self, x, cu, counts, w13, w2, row_scale, y, stage, ws, stream=None) -> None:
        """One grouped-FFN call on the weights ``set_weights`` prepared."""
        if self.w8a8:
            # x = (codes [rows, H], scales [H/128, stride], scale_src or None)
            xq, xs, src = x
            ops.moe_grouped_ffn_w8a8(xq, xs, cu, counts, w13[0], w13[1], w2[0], w2[1], row_scale,
                                     y, stage, ws, self.dev_error, stream=stream, scale_src=src,
                                     scale_div=self.K)
        elif self.fp8_weights:
            ops.moe_grouped_ffn_fp8(x, cu, counts, w13[0], w13[1], w2[0], w2[1], row_scale, y,
                                    stage, ws, self.dev_error, stream=stream)
        else:
            layout = ops.MOE_FFN_PACKED_WEIGHTS if self.packed else 0
            ops.moe_grouped_ffn(x, cu, counts, w13, w2, row_scale, y, stage | layout, ws,
                                self.dev_error, stream=stream)

    # ------------------------------------------------------------------ stages
    def stages(self, logits: torch.Tensor, hidden: torch.Tensor,
               row_valid: Optional[torch.Tensor] = None,
               overlap_shared: bool = False) -> List[Tuple[str, Callable[[], None]]]:
        """The layer as an ordered list of ``(name, enqueue)`` stages.  Each
        enqueue only launches kernels on the current stream; running a stage
        again with the same inputs rewrites the same outputs.  With
        ``overlap_shared`` the shared expert is the first stage instead and
        runs on the side stream, which the current stream waits for before
        the combine (the form ``forward`` uses; a graph capture of it holds
        the two branches)."""
        p = self.perm
        x = self.hidden_q if self.hidden_q is not None else hidden
        st = [("route", lambda: ops.moe_route(logits, self.K, row_valid, self.renormalize,
                                               self.topk_idx, self.topk_w))]
        if self.w8a8:
            # the dispatch quantizer for real: codes + scales of the [T, H]
            # rows; the permute moves the codes, the GEMM finds each permuted
            # row's scales through src_of
            x = self.hq.view(torch.bfloat16)
            x_ffn = (p.x_perm.view(torch.uint8), self.hs, p.src_of)
            x_shared = (self.hq, self.hs, None)
            st.append(("dispatch_quant", lambda: ops.moe_quant_rows_fp8(
                hidden, None, self.hq, self.hs)))
        else:
            x_ffn = p.x_perm
            x_shared = hidden
        if self.w8a8:
            pass                          # replaced by the real quantizer above
        elif self.dispatch_fp4:
            mode, block = _FP4[self.dispatch_fp4]
            st.append(("dispatch_qdq", lambda: ops.moe_fake_quant_rows(
                hidden, self.hidden_q, None, mode, block, self.dispatch_scale)))
        elif self.dispatch_block and not self.fuse_dispatch:
            st.append(("dispatch_qdq", lambda: ops.moe_fake_quant_rows(
                hidden, self.hidden_q, None, ops.MOE_FQ_BLOCK, self.dispatch_block)))
        fuse = self.fuse_dispatch and not self.w8a8
        st.append(("permute", lambda: ops.moe_permute(
            self.topk_idx, self.topk_w, x, self.El, self.expert_begin, self.pad_pow2,
            self.capacity, p, self.perm_ws, self.dev_error, dispatch_fp8=fuse,
            num_experts=self.E)))
        st.append(("ffn_gate_up", lambda: self._ffn(
            x_ffn, p.cu_seqlens, p.counts, self.w13, self.w2, p.w_perm, self.y_perm,
            ops.MOE_FFN_GATE_UP, self.ffn_ws)))
        st.append(("ffn_down", lambda: self._ffn(
            x_ffn, p.cu_seqlens, p.counts, self.w13, self.w2, p.w_perm, self.y_perm,
            ops.MOE_FFN_DOWN, self.ffn_ws)))
        if self.combine_fp4:
            # FP4 combine rows: the routed rows quantized in place (padding
            # rows skipped through src_of), then a plain combine
            cmode, cblock = _FP4[self.combine_fp4]
            st.append(("combine_qdq", lambda: ops.moe_fake_quant_rows(
                self.y_perm, self.y_perm, p.src_of, cmode, cblock, self.combine_scale)))
        if self.shared_I:
            def shared(stream=None):
                self._ffn(x_shared, self.shared_cu, self.shared_counts, self.shared_w13,
                          self.shared_w2, None, self.shared_out, ops.MOE_FFN_ALL,
                          self.shared_ws, stream=stream)

            if overlap_shared:
                def fork():
                    self.side.wait_stream(torch.cuda.current_stream())
                    shared(self.side)

                # it forks at the start, or (FP8 path) once its input rows
                # are quantized; the side stream waits for what precedes it
                at = [n for n, _ in st].index("dispatch_quant") + 1 if self.w8a8 else 0
                st.insert(at, ("shared_ffn", fork))
                st.append(("join_shared", lambda: torch.cuda.current_stream().wait_stream(self.side)))
            else:
                st.append(("shared_ffn", shared))
        fp8_scale = self.combine_scale if (self.combine_qdq and not self.combine_fp4) else None
        st.append(("combine", lambda: ops.moe_combine(
            self.y_perm, p.row_of, self.T, self.K, self.shared_out, fp8_scale, self.out,
            self.dev_error)))
        return st

    def forward(self, logits: torch.Tensor, hidden: torch.Tensor,
                row_valid: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Run the whole layer (enqueue only; no sync, no allocation), the
        shared expert concurrently with the routed path."""
        for _, enqueue in self.stages(logits, hidden, row_valid, overlap_shared=True):
            enqueue()
        return self.out

    def calibrate_combine_scale(self, logits, hidden, row_valid=None) -> torch.Tensor:
        """One-time max calibration of the constant combine-row scale: run the
        layer without combine-row QDQ, take max|row| over the routed rows and
        amax/448 (FP8) or amax/(6*448) (NVFP4) into the device scalar, all on
        the device (``moe_scale_from_amax``): no host round trip."""
        qdq, fp4 = self.combine_qdq, self.combine_fp4
        self.combine_qdq, self.combine_fp4 = False, None
        self.forward(logits, hidden, row_valid)
        self.combine_qdq, self.combine_fp4 = qdq, fp4
        self.amax.zero_()
        ops.moe_fake_quant_rows(self.y_perm, None, self.perm.src_of, ops.MOE_FQ_PER_TENSOR,
                                128, None, None, self.amax)
        if self.combine_scale is None:
            self.combine_scale = torch.zeros(1, dtype=torch.float32, device=self.device)
        mode = ops.MOE_FQ_NVFP4 if self.combine_fp4 == "nvfp4" else ops.MOE_FQ_PER_TENSOR
        ops.moe_scale_from_amax(self.amax, self.combine_scale, mode=mode)
        return self.combine_scale

    def stage_outputs(self) -> Dict[str, torch.Tensor]:
        p = self.perm
        d = dict(topk_idx=self.topk_idx, topk_w=self.topk_w, counts=p.counts,
                 cu_seqlens=p.cu_seqlens, x_perm=p.x_perm, row_of=p.row_of, src_of=p.src_of,
                 w_perm=p.w_perm, y_perm=self.y_perm, out=self.out)
        if self.hidden_q is not None:
            d["hidden_q"] = self.hidden_q
        if self.w8a8:
            d["hidden_codes"], d["hidden_scales"] = self.hq, self.hs
        if self.shared_out is not None:
            d["shared"] = self.shared_out
        return d
