#!/usr/bin/env python3
"""Throughput of the MoE-layer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
route -> (dispatch FP8 fake-quant) -> permute -> grouped SwiGLU FFN (gate/up
then down, BF16 MFMA) -> (shared expert) -> combine (+ combine-row FP8
fake-quant).  Inputs and weights are resident in HBM before timing starts.

Prints ONE JSON line: routed tokens/s for the layer, the roofline of the
dominant kernel (timed with HIP events on the stream it runs on), per-stage
times / achieved GB/s / MFMA utilisation, and the CPU oracle timed on a
bounded sample on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense BF16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic(cfg, counts: np.ndarray, fp8=None) -> dict:
    """Bytes (and FLOPs) each stage must move (compute) at minimum: every
    input read once, every output written once, padding rows and re-reads
    not counted.  FP8 weights (``fp8`` = "weights" or "w8a8"): one byte per
    weight plus a float32 scale per 128 x 128 tile; the FP8 path ("w8a8")
    also moves the rows and the intermediate as one-byte codes plus a float32
    scale per 1 x 128 block."""
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    Tv = cfg.T_valid
    N = int(counts.sum())
    E_act = int((counts > 0).sum())
    w8a8 = fp8 == "w8a8"
    st = {}
    st["route"] = dict(bytes=4 * T * E + 8 * T * K + (T if cfg.pad_rows else 0))
    if w8a8:
        st["dispatch_quant"] = dict(bytes=2 * T * H + T * H + T * H // 32)
    elif cfg.dispatch_block and cfg.dispatch_block != 128:
        st["dispatch_qdq"] = dict(bytes=4 * Tv * H)
    # (the 1 x 128 FP8 dispatch quantizer runs inside the permute, whose
    # bytes are unchanged: each valid token row is still read once)
    xb = 1 if w8a8 else 2                                  # bytes per row element
    st["permute"] = dict(bytes=8 * T * K + xb * Tv * H + xb * N * H + 4 * T * K + 8 * N + 8 * E)
    wb = 1 + 4 / (128 * 128) if fp8 else 2                 # bytes per weight
    if w8a8:
        st["ffn_gate_up"] = dict(bytes=int(wb * 2 * E_act * I * H) + N * H + N * H // 32 + 4 * N
                                 + N * I + N * I // 32, flops=4 * N * I * H)
        st["ffn_down"] = dict(bytes=int(wb * E_act * I * H) + N * I + N * I // 32 + 2 * N * H
                              + 4 * N, flops=2 * N * I * H)
    else:
        st["ffn_gate_up"] = dict(bytes=int(wb * 2 * E_act * I * H) + 2 * N * H + 2 * N * I,
                                 flops=4 * N * I * H)
        st["ffn_down"] = dict(bytes=int(wb * E_act * I * H) + 2 * N * I + 2 * N * H + 4 * N,
                              flops=2 * N * I * H)
    if cfg.shared_I:
        Is = cfg.shared_I
        st["shared_ffn"] = dict(bytes=int(wb * 3 * Is * H) + xb * T * H + 2 * T * H,
                                flops=6 * T * Is * H)
    st["combine"] = dict(bytes=2 * N * H + 4 * T * K + 2 * T * H + (2 * T * H if cfg.shared_I else 0))
    return st


STAGE_SOURCES = {
    "route": ["route.hip"], "dispatch_qdq": ["fake_quant.hip"], "permute": ["permute.hip"],
    "dispatch_quant": ["fp8_ffn.hip"], "combine": ["combine.hip"],
}
# the grouped GEMMs: the BF16 and FP8-weight kernels, or the FP8 path's
GEMM_SOURCES = {None: ["grouped_ffn.hip", "gemm_common.h"],
                "weights": ["grouped_ffn.hip", "gemm_common.h"],
                "w8a8": ["fp8_ffn.hip", "gemm_common.h"]}


def kernel_source_hash(stage: str, fp8=None) -> str:
    """Hash of the sources a stage's kernels are built from (plus common.h),
    for the weight/activation mode ``fp8`` (None, "weights" or "w8a8")."""
    names = STAGE_SOURCES.get(stage) or GEMM_SOURCES[fp8]
    h = hashlib.sha256()
    for name in names + ["common.h"]:
        with open(os.path.join(ROOT, "combine_top_route_moe_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def gemm_kernel_name(layer, fp8, gate_up: bool) -> str:
    """The grouped-GEMM kernel a routed projection launches: the FP8 path's,
    or, for segments averaging 96..255 rows (BF16 or FP8 weights), the
    streamed tall-tile kernel, else the fragment-streaming one.  The same
    rule as the library's launcher."""
    t = "true" if gate_up else "false"
    if fp8 == "w8a8":
        return f"w8a8_gemm_kernel<{t}>"
    mean = layer.capacity // layer.El
    if 96 <= mean < 256:
        return f"tall_stream_kernel<{t}>"
    return f"frag_gemm_kernel<{t}>"


def committed_traffic(stage: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the kernel as it is now (same source hash); else None.
    ``workload`` names the summary (the workload, plus "_fp8w" for FP8
    weights or "_w8a8" for the FP8 path)."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f).get(stage)
    fp8 = "w8a8" if workload.endswith("_w8a8") else "weights" if workload.endswith("_fp8w") else None
    if not d or d.get("source_hash") != kernel_source_hash(stage, fp8):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, logits, hidden, row_valid, budget_s: float, expert_weights, shared):
    """Time the oracle layer (as it stands) on a bounded sample of the batch:
    its first n tokens, n doubled from 8 until one run takes about a quarter
    of the budget, then repeated (median kept) until about half of it.

    ``expert_weights(e)`` returns expert e's bf16 weights as host arrays; the
    bench hands over a copy from the device tensors it uploaded (a few ms per
    expert, inside the timed oracle run), so no second copy of every
    expert's weights is held in host memory.  The sample is a prefix of the
    batch, so it pays the oracle's per-expert costs (converting each touched
    expert's weights to float64) for fewer tokens than the full batch would:
    the rate is a lower bound for the full batch, labelled as a sample."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
        if blas:
            cores = min(cores, max(blas))
    except Exception:
        pass

    def run(n):
        rv = None if row_valid is None else row_valid[:n]
        t0 = time.perf_counter()
        oracle.moe_layer(logits[:n], hidden[:n], expert_weights, cfg.K, rv,
                         dispatch_block=cfg.dispatch_block or None, pad_pow2=cfg.pad_pow2,
                         shared_weights=shared, combine_qdq=cfg.combine_qdq)
        return time.perf_counter() - t0

    n = min(cfg.T, 8)
    dt = run(n)
    while n < cfg.T and dt < budget_s / 4:
        n = min(cfg.T, n * 2)
        dt = run(n)
    times = [dt]
    while sum(times) < budget_s / 2 and len(times) < 50:
        times.append(run(n))
    dt = float(np.median(times))
    tv = n if row_valid is None else int(row_valid[:n].sum())
    touched = len(set(int(e) for e in oracle.route(logits[:n], None if row_valid is None
                                                   else row_valid[:n], cfg.K)[0].reshape(-1)
                      if e >= 0))
    return {"value": tv / dt, "unit": "routed tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens of the {cfg.name} batch ({tv} routed, "
                      f"{touched} of {cfg.E} experts touched), whole layer, float64 numpy, "
                      f"median of {len(times)} runs: {dt:.2f} s; a prefix pays each touched "
                      "expert's weight conversion for fewer tokens than the whole batch, so "
                      "this sampled rate is a lower bound for the full batch"}


def calibrate_spin(stream, target_ms: float = 1.0) -> int:
    """Cycles for torch.cuda._sleep to keep the GPU busy about target_ms."""
    import torch

    cycles = 1 << 20
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(cycles)
    b.record(stream)
    torch.cuda.synchronize()
    ms = max(a.elapsed_time(b), 1e-3)
    return int(cycles * target_ms / ms)


def copy_gbps(steps: int = 5, nbytes: int = 1 << 30) -> float:
    """Bandwidth of moe_copy_bytes (read + write) over 1 GiB: the plain
    16-byte streaming copy, timed with events on the launch stream."""
    import torch
    from combine_top_route_moe_amd import ops

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    ops.moe_copy_bytes(src, dst)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        ops.moe_copy_bytes(src, dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def read_gbps(steps: int = 5, nbytes: int = 1 << 30) -> float:
    """Bandwidth of moe_read_bytes over 1 GiB of random bytes: the plain
    non-temporal read stream (the practical ceiling of the weight-streaming
    GEMMs), timed with events on the launch stream."""
    import torch
    from combine_top_route_moe_amd import ops

    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    ops.moe_read_bytes(src, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        ops.moe_read_bytes(src, sink)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del src, sink
    return nbytes / (ms * 1e-3) / 1e9


def copy_calibration(steps: int, warmup: int) -> None:
    """Time moe_copy_bytes over 1 GiB: the plain streaming kernel whose
    measured bandwidth and FETCH_SIZE / WRITE_SIZE counters calibrate the
    other kernels' figures (it reads and writes exactly 1 GiB per launch)."""
    import torch
    from combine_top_route_moe_amd import ops

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(warmup):
        ops.moe_copy_bytes(src, dst)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        ops.moe_copy_bytes(src, dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"kernel": "copy_kernel", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "ms_per_launch": round(ms, 4),
                      "GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def pct(v, q):
    return round(float(np.percentile(np.asarray(v, dtype=np.float64), q)), 5)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="deepseek",
                    help="deepseek (default: the largest workload) | prefill | balanced | "
                         "skewed | tiny")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold-stages", action="store_true",
                    help="skip the stage timing with 1 GiB written before every step (cold "
                         "caches), reported as stages_cold")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the steps as eager launches instead of HIP-graph replays")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time")
    ap.add_argument("--fp8", choices=["weights", "w8a8"], default=None,
                    help="weights: expert weights as E4M3 codes with 128x128 tile scales, "
                         "dequantized in registers before the BF16 MFMAs; w8a8: rows and weights "
                         "as E4M3 codes on the FP8 matrix cores")
    ap.add_argument("--fp8-weights", action="store_const", const="weights", dest="fp8",
                    help="same as --fp8 weights")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the reference copy kernel (1 GiB -> 1 GiB) and report its "
                         "bandwidth; its byte counters scale the PMC traffic figures")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the MoE layer here runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU expert-parallel exchange is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from combine_top_route_moe_amd import MoELayer, ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        copy_calibration(args.steps, args.warmup)
        return
    cfg = workloads.CONFIGS[args.config]
    if ops.moe_device_check(0) != 0:
        raise SystemExit("device 0 is not a gfx950 GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    logits_h = workloads.logits(cfg)
    hidden_h = workloads.hidden(cfg)
    valid_h = workloads.row_valid(cfg)
    logits = torch.from_numpy(logits_h).to(dev)
    hidden = bf16(hidden_h)
    row_valid = None if valid_h is None else torch.from_numpy(valid_h).to(dev)

    layer = MoELayer(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, dev, shared_I=cfg.shared_I,
                     dispatch_block=cfg.dispatch_block, combine_qdq=cfg.combine_qdq,
                     pad_pow2=cfg.pad_pow2)
    w13 = torch.empty(cfg.E, 2 * cfg.I, cfg.H, dtype=torch.bfloat16, device=dev)
    w2 = torch.empty(cfg.E, cfg.H, cfg.I, dtype=torch.bfloat16, device=dev)

    def put(e, a, b):
        w13[e].copy_(bf16(a))
        w2[e].copy_(bf16(b))

    workloads.for_each_expert(cfg, put)
    sw = workloads.shared_weights(cfg)
    layer.set_weights(w13, w2, *(bf16(x) for x in sw) if sw else (None, None),
                      fp8={None: False, "weights": True, "w8a8": "w8a8"}[args.fp8])
    if args.fp8 or args.no_cpu_baseline:
        del w13, w2                   # only the packed weights stay resident
    if cfg.combine_qdq:
        layer.calibrate_combine_scale(logits, hidden, row_valid)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        layer.forward(logits, hidden, row_valid)
    torch.cuda.synchronize()
    layer.dev_error.zero_()
    stream = torch.cuda.current_stream()

    # Timed region 1 (value, ms_per_step): K whole-layer steps.  By default
    # the layer is captured once into a HIP graph and replayed (every entry
    # point is capture-safe: no host sync, no allocation); --no-graph times
    # eager launches instead.
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            layer.forward(logits, hidden, row_valid)
        stream.wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layer.forward(logits, hidden, row_valid)
        for _ in range(args.warmup):
            graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            layer.forward(logits, hidden, row_valid)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert layer.dev_error.item() == 0, "device error word set during the timed run"

    # Per-step layer times (after the timed region, not instead of it): each
    # graph replay and each eager step bracketed by events on the launch
    # stream, for the median and the p10 / p90 spread.
    def per_step(fn):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(args.steps):
            fn()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        return [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]

    layer_ms = {}
    if graph is not None:
        layer_ms["graph"] = per_step(graph.replay)
    layer_ms["eager"] = per_step(lambda: layer.forward(logits, hidden, row_valid))

    # Timed region 2 (stages, roofline): K eager steps with HIP events between
    # the stages on the launch stream.  Each step is preceded by a short GPU
    # spin kernel, so the host has enqueued the whole step (and its events)
    # before the GPU reaches it: the stages then run back to back, with the
    # cache state of a real step, and the events time GPU work only.
    stages = layer.stages(logits, hidden, row_valid)
    spin_cycles = calibrate_spin(stream)

    def time_stages(flush=None):
        per_stage = {name: [] for name, _ in stages}
        for _ in range(args.steps):
            if flush is not None:
                flush.fill_(1)             # evicts L2 and the infinity cache
            torch.cuda._sleep(spin_cycles)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
            evs[0].record(stream)
            for i, (name, enqueue) in enumerate(stages):
                enqueue()
                evs[i + 1].record(stream)
            torch.cuda.synchronize()
            for i, (name, _) in enumerate(stages):
                per_stage[name].append(evs[i].elapsed_time(evs[i + 1]))
        return per_stage

    stage_samples = time_stages()
    # Timed region 3 (stages_cold): the same with 1 GiB written before every
    # step, so each stage starts from cold L2 and infinity cache (a replayed
    # layer otherwise finds part of its weights, and the small workloads part
    # of their rows, in the infinity cache); reported beside the in-context
    # figures, not instead of them.  --no-cold-stages skips it (the profiled
    # runs do, so that their kernel averages are the in-context launches).
    stage_samples_cold = None
    if not args.no_cold_stages:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        stage_samples_cold = time_stages(flush)
        del flush
    assert layer.dev_error.item() == 0, "device error word set during the stage timing"
    copy_bw = copy_gbps()
    read_bw = read_gbps()

    counts = layer.perm.counts.cpu().numpy()
    alg = algorithmic(cfg, counts, args.fp8)
    peak_mfma = PEAK_FP8_TFLOPS if args.fp8 == "w8a8" else PEAK_BF16_TFLOPS

    def stage_report(samples):
        out = {}
        for name, v in samples.items():
            ms = float(np.median(v))
            a = alg.get(name, {})
            d = {"ms": round(ms, 5), "ms_p10": pct(v, 10), "ms_p90": pct(v, 90)}
            if "bytes" in a:
                d["alg_bytes"] = a["bytes"]
                d["GBps"] = round(a["bytes"] / (ms * 1e-3) / 1e9, 1)
                d["hbm_frac"] = round(d["GBps"] / PEAK_HBM_GBPS, 4)
            if "flops" in a:
                d["TFLOPs"] = round(a["flops"] / (ms * 1e-3) / 1e12, 2)
                d["mfma_util"] = round(d["TFLOPs"] / peak_mfma, 4)
            out[name] = d
        return out

    stage_ms = {k: float(np.median(v)) for k, v in stage_samples.items()}
    stages = stage_report(stage_samples)
    stages_cold = stage_report(stage_samples_cold) if stage_samples_cold else None

    dom = max(stage_ms, key=stage_ms.get)
    a = alg[dom]
    intensity = a.get("flops", 0) / a["bytes"]
    ridge = peak_mfma * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": stages[dom]["TFLOPs"], "peak": peak_mfma,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": stages[dom]["GBps"], "peak": PEAK_HBM_GBPS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = {"ffn_gate_up": gemm_kernel_name(layer, args.fp8, True),
                      "ffn_down": gemm_kernel_name(layer, args.fp8, False)}.get(dom, dom)
    roof["alg_bytes_per_launch"] = a["bytes"]
    roof["traffic"] = committed_traffic(
        dom, cfg.name + {None: "", "weights": "_fp8w", "w8a8": "_w8a8"}[args.fp8])

    ms_step = elapsed / args.steps * 1e3
    gemm_flops = alg["ffn_gate_up"]["flops"] + alg["ffn_down"]["flops"]
    gemm_ms = stage_ms["ffn_gate_up"] + stage_ms["ffn_down"]
    result = {
        "metric": "routed tokens/sec per MoE layer; grouped-GEMM MFMA util; permute/combine GB/s",
        "value": round(cfg.T_valid / (elapsed / args.steps), 1),
        "unit": "routed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if args.fp8 == "w8a8" else "bf16",
        "data": "synthetic (seeded N(0,1) logits and hidden, N(0,0.02) weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "T_valid": cfg.T_valid, "H": cfg.H,
                   "E": cfg.E, "K": cfg.K, "I": cfg.I, "shared_I": cfg.shared_I,
                   "routed_rows": int(counts.sum()), "dispatch_fp8_block": cfg.dispatch_block,
                   "combine_fp8": cfg.combine_qdq, "pad_pow2": cfg.pad_pow2,
                   "expert_weights": ("fp8 e4m3, 128x128 tile scales" if args.fp8
                                      else "bf16"),
                   "activations": ("fp8 e4m3, 1x128 block scales" if args.fp8 == "w8a8"
                                   else "bf16"),
                   "parallelism": "single GPU (all experts local)"},
        "grouped_gemm_mfma_util": round(gemm_flops / (gemm_ms * 1e-3) / (peak_mfma * 1e12), 4),
        "permute_GBps": stages["permute"]["GBps"],
        "combine_GBps": stages["combine"]["GBps"],
        "copy_GBps": round(copy_bw, 1),
        "read_GBps": round(read_bw, 1),
        "layer_ms": {k: {"median": round(float(np.median(v)), 5), "p10": pct(v, 10),
                         "p90": pct(v, 90)} for k, v in layer_ms.items()},
        "stages": stages,
        **({"stages_cold": stages_cold} if stages_cold else {}),
        "roofline": roof,
        "timing": {"value": ("HIP-graph replay of the whole layer" if graph is not None
                             else "eager launches of the whole layer"),
                   "layer_ms": "each graph replay and each eager whole-layer step between HIP "
                               "events on the launch stream (after the timed region)",
                   "stages": "eager steps queued behind a GPU spin kernel, HIP events between "
                             "stages on the launch stream, median (p10, p90) over steps; stages "
                             "run one after another (the layer itself runs the shared expert "
                             "concurrently with the routed path)",
                   "copy_GBps": "moe_copy_bytes, 1 GiB read + 1 GiB written per launch",
                   "read_GBps": "moe_read_bytes, 1 GiB of random bytes read per launch",
                   **({"stages_cold": "the same, with 1 GiB written before every step "
                                      "(cold L2 and infinity cache)"} if stages_cold else {})},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        if args.fp8:
            result["cpu_baseline_note"] = (
                "not timed in the FP8 modes: the oracle quantizes each expert's weights to "
                "128 x 128 tiles in numpy (seconds per expert), which a bounded sample cannot "
                "separate from the layer; the BF16 line carries the oracle baseline")
        else:
            def expert_weights(e):
                return (w13[e].view(torch.int16).cpu().numpy().view(np.uint16),
                        w2[e].view(torch.int16).cpu().numpy().view(np.uint16))

            result["cpu_baseline"] = cpu_baseline(cfg, logits_h, hidden_h, valid_h,
                                                  args.cpu_budget, expert_weights, sw)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
