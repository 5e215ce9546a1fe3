"""Host checks of the measurement harness and of the product/oracle split
(no GPU needed).

* ``bench.py --gpus N`` with N > 1 refuses with a message (one GPU only).
* The algorithmic byte and FLOP counts that the roofline figures divide by
  follow their formulas: on the balanced shape with 64 rows per expert,
  permute 8TK + 2 T_v H + 2NH + 4TK + 8N + 8E = 18.96 MB, combine
  2NH + 4TK + 2TH = 18.89 MB, grouped FFN 6NIH = 51.5 GFLOP and weight bytes
  2 * 3 E I H = 805 MB.
* The product package never refers to the oracle (only tests, smoke() and
  the bench's CPU baseline may).
"""

import os
import re
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_algorithmic_counts_balanced():
    import bench
    import workloads

    cfg = workloads.CONFIGS["balanced"]
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    counts = np.full(E, T * K // E, dtype=np.int64)           # 64 rows per expert
    N = T * K
    st = bench.algorithmic(cfg, counts)
    assert st["permute"]["bytes"] == 8 * T * K + 2 * T * H + 2 * N * H + 4 * T * K + 8 * N + 8 * E
    assert abs(st["permute"]["bytes"] / 1e6 - 18.96) < 0.01
    assert st["combine"]["bytes"] == 2 * N * H + 4 * T * K + 2 * T * H
    assert abs(st["combine"]["bytes"] / 1e6 - 18.89) < 0.01
    flops = st["ffn_gate_up"]["flops"] + st["ffn_down"]["flops"]
    assert flops == 6 * N * I * H
    assert abs(flops / 1e9 - 51.5) < 0.1
    weight_bytes = 2 * 2 * E * I * H + 2 * E * I * H
    assert st["ffn_gate_up"]["bytes"] + st["ffn_down"]["bytes"] == (
        weight_bytes + 2 * N * H + 2 * N * I + 2 * N * I + 2 * N * H + 4 * N)
    # FP8 weights: one byte per weight plus a float32 scale per 128 x 128 tile
    st8 = bench.algorithmic(cfg, counts, "weights")
    w8 = int((1 + 4 / (128 * 128)) * 2 * E * I * H) + int((1 + 4 / (128 * 128)) * E * I * H)
    assert st8["ffn_gate_up"]["bytes"] + st8["ffn_down"]["bytes"] == (
        w8 + 2 * N * H + 2 * N * I + 2 * N * I + 2 * N * H + 4 * N)


def test_product_package_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "combine_top_route_moe_amd")
    for dirpath, _, files in os.walk(pkg):
        for name in files:
            if name.endswith((".py", ".hip", ".h", ".cpp")):
                with open(os.path.join(dirpath, name)) as f:
                    text = f.read()
                assert not re.search(r"\boracle\b", text), os.path.join(dirpath, name)
