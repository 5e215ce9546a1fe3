"""CPU oracle for the MoE-layer hot path — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition of what the
GPU path computes: route → (dispatch fake-quant) → permute → grouped SwiGLU
FFN → (combine-row fake-quant) → ordered combine.  It is written from the
four pages the method comes from, each function citing the passage it
follows, and it shares no code with the HIP library: no kernels, headers,
tables or constants are common to the two.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product path (the C-ABI library and
its Python binding) never calls into it.

Precision: everything the pages fix exactly is emulated exactly (IEEE
binary32 adds in the combine, one bfloat16 round-to-nearest-even, OCP
E4M3FN and E2M1 round-to-nearest-even with saturation).  Everything else (softmax
weights, the expert FFN) is computed in float64.

Pins (tests/test_oracle_*.py, run with ``-m "not gpu"``) tie every function
here to something other than itself: library casts (torch CPU bfloat16 and
float8_e4m3fn), brute force on tiny inputs, closed forms and hand-worked
examples.  A function with no such pin would say "parity unpinned" here;
there is none at present.
"""

from .numerics import (
    bf16_bits_to_f64,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    e4m3fn_table,
    e4m3fn_round,
    qdq_e4m3fn,
)
from .route import route
from .quant import fake_quant_block, fake_quant_per_tensor, calibrate_amax, quantize_weight_blocks
from .fp4 import e2m1_round, fake_quant_mxfp4, fake_quant_nvfp4, nvfp4_tensor_scale
from .permute import permute, next_pow2
from .ffn import expert_ffn, grouped_ffn
from .fp8_gemm import (quantize_rows_fp8, block_scaled_matmul, expert_ffn_w8a8,
                       expert_ffn_w8a8_steps, grouped_ffn_w8a8)
from .combine import combine
from .layer import moe_layer

__all__ = [
    "bf16_bits_to_f64", "bf16_bits_to_f32", "f32_to_bf16_bits",
    "e4m3fn_table", "e4m3fn_round", "qdq_e4m3fn",
    "route", "fake_quant_block", "fake_quant_per_tensor", "calibrate_amax",
    "permute", "next_pow2", "expert_ffn", "grouped_ffn", "combine", "moe_layer",
    "quantize_weight_blocks", "quantize_rows_fp8", "block_scaled_matmul", "expert_ffn_w8a8",
    "expert_ffn_w8a8_steps", "grouped_ffn_w8a8",
]
