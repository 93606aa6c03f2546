"""Benchmark of the parallel-block forward on one MI355X.

One step = one pass of the whole hot path (LayerNorm, fused QKV+FC1 GEMM with
the GeLU epilogue, sliding-window attention, fused out-proj+FC2 GEMM) over one
batch of seeded synthetic input already resident in HBM.  Default workload:
one 1/8 tensor-parallel shard of the 175B layer (B=1, S=2048, d=12288, 12
local heads x 128, local ffn 6144, W=512), emitting the pre-reduce-scatter
partial.

Prints ONE JSON line: throughput in TFLOP/s of algorithmic work, % of the bf16
MFMA peak, tokens/s, per-kernel times measured with HIP events inside the
timed region, the roofline record of the dominant kernel, and the fp64 CPU
oracle timed on the host as a baseline.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload shard175b]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "parallel-block fwd TFLOP/s and % of bf16 MFMA peak; tokens/s (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0      # MI355X published HBM3E bandwidth
DEFAULT_WORKLOAD = "shard175b"

# HBM traffic of the dominant kernel from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# runs, scaled by the same counters read on a plain copy of known size.  Bytes
# per launch; None until measured for the current kernel build.
MEASURED_TRAFFIC_BYTES = {
    # gemm_in main kernel + its split-K tail reduce (profiles/shard175b_kernels.md); set
    # only for the GEMM build the counters were taken on (4-wave 128x128, 64-deep slabs)
    "shard175b": 1025501926,
}

WORKLOAD_NOTES = {
    "shard175b": "1/8 tensor-parallel shard of the 175B layer (hidden 12288, TP 8), one GPU; output is the "
                 "pre-reduce-scatter partial (no residual)",
    "small": "small block", "long": "long sequence, 1024-key window", "fullcausal": "window covers the sequence",
    "tiny": "tiny fp32 debug block",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on the host")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (for HBM counter calibration) and exit")
    return p.parse_args()


def copy_calibration(mib: int) -> None:
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}), flush=True)


def cpu_baseline(cfg, inp) -> dict:
    """The fp64 oracle, as it stands, timed once on the host cores over the whole workload."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W, eps=cfg.ln_eps,
                         add_residual=bool(cfg.add_residual))
    dt = time.perf_counter() - t0
    return {"value": round(cfg.flops() / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3), "tokens_per_s": round(cfg.M / dt, 1),
            "sample": f"one full forward of the {cfg.name} workload (all {cfg.M} tokens), float64 numpy"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: this build runs on one GPU only (asked for {max(args.gpus, world)}); the block is "
              "measured on one GPU's share at its real shape. Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import transformer_block_fwd_amd as tb
    from workload import CONFIGS, make_inputs

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    cfg = CONFIGS[args.workload]
    print(f"[bench] workload {cfg}", file=sys.stderr, flush=True)
    inp = make_inputs(cfg, seed=0)
    arrs = inp.device_arrays()
    if cfg.dtype == "bf16":
        dev = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).cuda()
               for k, v in arrs.items()}
    else:
        dev = {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda() for k, v in arrs.items()}
    out = torch.empty_like(dev["x"])
    weights = (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"])
    stream = torch.cuda.current_stream()
    h = tb.pblock_create(cfg)

    for _ in range(args.warmup):
        tb.pblock_forward(h, dev["x"], weights, cfg, out, stream)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    tb.pblock_set_timing(h, True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        tb.pblock_forward(h, dev["x"], weights, cfg, out, stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(end)
    kernel_ms, n_fwd = tb.pblock_kernel_times(h)
    tb.pblock_set_timing(h, False)
    print(f"[bench] timed {args.steps} steps in {ms_total:.3f} ms (wall {wall * 1e3:.3f} ms)", file=sys.stderr,
          flush=True)

    ms_step = ms_total / args.steps
    flops = cfg.flops()
    tflops = flops / (ms_step * 1e-3) / 1e12
    k_avg = {k: v / max(n_fwd, 1) for k, v in kernel_ms.items()}
    g1_ms = k_avg["gemm_in"]
    g1_tflops = cfg.gemm1_flops() / (g1_ms * 1e-3) / 1e12
    traffic = MEASURED_TRAFFIC_BYTES.get(cfg.name)
    roofline = {"kernel": "gemm_in (fused QKV+FC1 GEMM, GeLU epilogue)", "bound": "mfma",
                "achieved": round(g1_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g1_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flops_per_launch": cfg.gemm1_flops(), "avg_launch_ms": round(g1_ms, 5)}
    per_kernel = {}
    for k, ms in k_avg.items():
        kf = {"gemm_in": cfg.gemm1_flops(), "gemm_out": cfg.gemm2_flops(), "attention": cfg.attn_flops()}.get(k)
        rec = {"ms": round(ms, 5)}
        if kf:
            rec["tflops"] = round(kf / (ms * 1e-3) / 1e12, 2)
        if k == "layernorm":
            es = 2 if cfg.dtype == "bf16" else 4
            rec["gbs"] = round((2 * cfg.M * cfg.d * es + 2 * cfg.d * es) / (ms * 1e-3) / 1e9, 1)
        per_kernel[k] = rec

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights)",
        "config": {"workload": f"{cfg.name}: {WORKLOAD_NOTES.get(cfg.name, '')}", "B": cfg.B, "S": cfg.S,
                   "d": cfg.d, "H": cfg.H, "hd": cfg.hd, "ffn": cfg.ffn, "W": cfg.W,
                   "add_residual": cfg.add_residual, "parallelism": "single GPU"},
        "pct_peak_bf16": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(cfg.M / (ms_step * 1e-3), 1),
        "algorithmic_gflop_per_step": round(flops / 1e9, 3),
        "kernels": per_kernel,
        "roofline": roofline,
    }
    tb.pblock_destroy(h)
    del dev, out
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, inp)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
