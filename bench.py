"""Benchmark of the parallel-block forward on one MI355X.

One step = one pass of the whole hot path (LayerNorm, fused QKV+FC1 GEMM with
the GeLU epilogue, sliding-window attention, fused out-proj+FC2 GEMM) over one
batch of seeded synthetic input already resident in HBM.  Default workload:
one 1/8 tensor-parallel shard of the 175B layer (B=1, S=2048, d=12288, 12
local heads x 128, local ffn 6144, W=512), emitting the pre-reduce-scatter
partial.

Order of a run: W warm-up steps, the timed region (exactly K steps between two
events: `value`, `ms_per_step`), then the same K steps again with HIP events
around every step and every kernel launch (`instrumented`: the per-step spread,
the per-kernel times and the roofline record of the dominant kernel), then the
other measurements.  From a cold start the forward needs about 30 steps to reach
its sustained rate (`--ramp` records that ramp step by step); the default 40
warm-up steps cover it, so `value` is the sustained rate (with fewer warm-up
steps the timed region includes part of the ramp).

Prints ONE JSON line: throughput in TFLOP/s of algorithmic work, % of the bf16
MFMA peak, tokens/s, the instrumented pass, a cold-cache pass, per-kernel times,
the roofline record, the MFMA-loop rate, and the fp64 CPU oracle timed on the
host as a baseline.

  python bench.py [--gpus 1] [--steps 50] [--warmup 40] [--workload shard175b]
                  [--block parallel|serial] [--window W] [--chunks N]
                  [--gelu-tanh] [--bias] [--rope BASE] [--two-ln]   # variant switches
                  [--train]    # forward with saved activations + backward pass
  python bench.py --sweep      # attention time against window and sequence length
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "parallel-block fwd TFLOP/s and % of bf16 MFMA peak; tokens/s (1 GPU)"
METRIC_TRAIN = "parallel-block training step (fwd + bwd) TFLOP/s and % of bf16 MFMA peak; tokens/s (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0      # MI355X published HBM3E bandwidth
DEFAULT_WORKLOAD = "shard175b"
COLD_SCRUB_MIB = 512       # written between cold-cache steps (more than the 256 MB last-level cache)

# HBM traffic of the dominant kernel from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# runs, scaled by the same counters read on a plain copy of known size.  Bytes
# per launch; None until measured for the current kernel build.
MEASURED_TRAFFIC_BYTES = {
    # gemm_in main kernel (profiles/shard175b_kernels.md; its split-K reduce runs in the attention
    # launch); set only for the GEMM build the counters were taken on (4-wave 128x128 as 16x16x32
    # MFMA tiles, 64-deep slabs, copies spread evenly over three phases, row-major split-K
    # partials, the direct lane-swap epilogue, the 5-term erfc GeLU as max(z, 0) - |z| h;
    # tile-height, tile-width, row-chunk publication and direct-epilogue template parameters at
    # 256, 256, off and on for this launch; the saved pre-activation store in that epilogue's
    # code, off for this launch)
    "shard175b": 950000518,
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
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--block", choices=("parallel", "serial"), default="parallel",
                   help="the parallel block (default) or the serial pre-LN layer from the same kernels")
    p.add_argument("--window", type=int, default=0, help="override the workload's attention window W")
    p.add_argument("--add-residual", type=int, choices=(0, 1), default=None,
                   help="override the workload's add_residual (the serial form always adds it)")
    p.add_argument("--chunks", type=int, default=0,
                   help="time the forward in this many position chunks (the TP/SP overlap form) with a completion "
                        "event per chunk; per-kernel and roofline figures then come from an unchunked pass")
    p.add_argument("--chunk-input", action="store_true",
                   help="with --chunks: pass per-chunk input events too (all steps chunked, the all-gather side "
                        "of the overlap); without it only the output GEMM is chunked")
    p.add_argument("--rowchunks", action="store_true",
                   help="with --chunks: one output-GEMM launch that publishes each chunk through a device flag "
                        "(pblock_forward_rowchunks) instead of one launch per chunk; one more step with the "
                        "consumer (pblock_pack_chunks) on a second stream reports the publication times")
    p.add_argument("--gelu-tanh", action="store_true", help="variant: tanh-form GeLU")
    p.add_argument("--bias", action="store_true", help="variant: biases on both projections")
    p.add_argument("--rope", type=float, default=0.0, metavar="BASE",
                   help="variant: rotary embedding of q and k with this base (0: off)")
    p.add_argument("--two-ln", action="store_true", help="variant: a second LayerNorm for the MLP branch")
    p.add_argument("--train", action="store_true",
                   help="time a training step: the forward that saves activations plus the backward pass")
    p.add_argument("--cold-steps", type=int, default=10, help="cold-cache steps after the timed run (0: skip)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on the host")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (for HBM counter calibration) and exit")
    p.add_argument("--ramp", action="store_true",
                   help="only measure from a cold start: per-step times of the forward over its first 120 steps "
                        "after 5 warm-up steps, then 60 steps each with the per-kernel timing events on, off, on")
    p.add_argument("--vs-torch-gemm", action="store_true",
                   help="only compare each workload's two GEMMs (the library's, epilogues included) with "
                        "torch.nn.functional.linear (hipBLASLt) on the same bf16 operands")
    p.add_argument("--sweep", action="store_true",
                   help="only time the attention kernel over windows and sequence lengths and fit time vs keys")
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


def backward_flops(cfg) -> float:
    """Algorithmic FLOPs of the backward pass: each GEMM twice (input and weight gradients) and
    the attention backward at 2.5x its forward (dV, dP, dQ, dK and the recomputed scores)."""
    return 2.0 * (cfg.gemm1_flops() + cfg.gemm2_flops()) + 2.5 * cfg.attn_flops()


CPU_BASELINE_MIN_S = 10.0  # the oracle is repeated until this much host time has been spent
CPU_BASELINE_MAX_RUNS = 10000


def cpu_baseline(cfg, inp, block, ln2, variant=None, train_dy=None) -> dict:
    """The fp64 oracle, as it stands, timed on the host cores over the whole workload: repeated
    until at least CPU_BASELINE_MIN_S seconds have passed, the median run reported."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1

    def run():
        if train_dy is not None:
            oracle.block_backward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, train_dy, cfg.H, cfg.hd, cfg.W,
                                  eps=cfg.ln_eps, add_residual=bool(cfg.add_residual))
        elif block == "serial":
            oracle.serial_block_forward(inp.x, inp.gamma, inp.beta, ln2["gamma2"], ln2["beta2"], inp.w_in,
                                        inp.w_out, cfg.H, cfg.hd, cfg.W, eps=cfg.ln_eps)
        elif variant is not None:
            oracle.block_forward_variant(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                                         eps=cfg.ln_eps, add_residual=bool(cfg.add_residual), **variant)
        else:
            oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                                 eps=cfg.ln_eps, add_residual=bool(cfg.add_residual))

    times = []
    while sum(times) < CPU_BASELINE_MIN_S and len(times) < CPU_BASELINE_MAX_RUNS:
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    dt = percentile(times, 0.5)
    what = "forward + backward" if train_dy is not None else "forward"
    fl = cfg.flops() + (backward_flops(cfg) if train_dy is not None else 0.0)
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3), "runs": len(times), "total_seconds": round(sum(times), 2),
            "tokens_per_s": round(cfg.M / dt, 1),
            "sample": f"the full {what} of the {cfg.name} workload (all {cfg.M} tokens), float64 numpy; "
                      f"{len(times)} run(s) in {sum(times):.1f} s, the median run"}


def percentile(v, q):
    s = sorted(v)
    k = (len(s) - 1) * q
    lo, hi = int(k), min(int(k) + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (k - lo)


def mfma_loop_rate(tb, torch, stream, form: str = "16x16x32") -> float:
    """TFLOP/s of the library's register-only MFMA loop over all CUs (about 20 ms), of the GEMMs'
    16x16x32 instruction or of the 32x32x16 one."""
    wgs = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    iters = 4000
    tb.pblock_mfma_loop(wgs, 100, sink, stream, form=form)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    tb.pblock_mfma_loop(wgs, iters, sink, stream, form=form)
    e.record(stream)
    torch.cuda.synchronize()
    return wgs * 4 * iters * 16 * 32768 / (s.elapsed_time(e) * 1e-3) / 1e12


def gemm_vs_torch() -> None:
    """Per bf16 workload: the library's input GEMM (with its GeLU epilogue and split-K tail) and
    output GEMM (with its tail launch) from its per-kernel events over 30 forwards after 40
    untimed ones, against torch.nn.functional.linear (hipBLASLt) on the same operand shapes and
    data, 30 calls each after 5 untimed ones (and after the library's forwards); algorithmic
    TFLOP/s of each."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    import transformer_block_fwd_amd as tb
    from workload import CONFIGS, make_inputs

    rows = []
    for name in ("small", "shard175b", "long", "fullcausal"):
        cfg = CONFIGS[name]
        inp = make_inputs(cfg, seed=0)
        dev = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).cuda()
               for k, v in inp.device_arrays().items()}
        w = (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"])
        out = torch.empty_like(dev["x"])
        h = tb.pblock_create(cfg)
        for _ in range(40):  # the warm-up the forward benchmark gives (clocks ramp over the first forwards)
            tb.pblock_forward(h, dev["x"], w, cfg, out)
        tb.pblock_set_timing(h, True)
        for _ in range(30):
            tb.pblock_forward(h, dev["x"], w, cfg, out)
        ms, n = tb.pblock_kernel_times(h)
        tb.pblock_set_timing(h, False)
        tb.pblock_destroy(h)
        M = cfg.M
        x2 = dev["x"].view(M, cfg.d)
        ag = torch.randn(M, cfg.k_out, device="cuda").to(torch.bfloat16)

        def t_linear(a, b, reps=30):
            for _ in range(5):
                F.linear(a, b)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                F.linear(a, b)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        t_in, t_out = t_linear(x2, dev["w_in"]), t_linear(ag, dev["w_out"])
        for gemm, ours, theirs, fl, shape in (
                ("in", ms["gemm_in"] / n, t_in, cfg.gemm1_flops(), (M, cfg.n_in, cfg.d)),
                ("out", ms["gemm_out"] / n, t_out, cfg.gemm2_flops(), (M, cfg.d, cfg.k_out))):
            rows.append({"workload": name, "gemm": gemm, "MxNxK": "x".join(map(str, shape)),
                         "library_ms": round(ours, 5), "library_tflops": round(fl / (ours * 1e-3) / 1e12, 1),
                         "torch_linear_ms": round(theirs, 5), "torch_linear_tflops": round(fl / (theirs * 1e-3) / 1e12, 1),
                         "library_over_torch_time": round(ours / theirs, 3)})
            print(f"[gemm] {name} {gemm} {rows[-1]['MxNxK']}: library {ours * 1e3:.1f} us, torch linear "
                  f"{theirs * 1e3:.1f} us", file=sys.stderr, flush=True)
        del dev, out, ag
        torch.cuda.empty_cache()
    print(json.dumps({"gemm_vs_torch_linear": rows,
                      "note": "library GEMMs include their epilogues (GeLU on FC1 columns; residual store) and tail "
                              "launches; torch linear is a plain bf16 GEMM"}), flush=True)


def attention_sweep() -> None:
    """Attention kernel time against the number of (query, key) pairs it must score:
    W in {128 .. 2048} at S = 8192 and S in {2048, 4096} at W = 1024 (the long
    workload's heads), a least-squares line through the points, and the full-causal
    workload's attention against that line's prediction."""
    import numpy as np
    import torch

    import transformer_block_fwd_amd as tb
    from workload import CONFIGS

    base = CONFIGS["long"]
    H, hd = base.H, base.hd
    A = H * hd
    torch.manual_seed(0)
    stream = torch.cuda.current_stream()

    def time_attention(B, S, W, reps=20):
        qkv = torch.randn(B * S, 3 * A, device="cuda", dtype=torch.bfloat16)
        o = torch.empty(B * S, A, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            tb.pblock_swa_attention(qkv, 3 * A, o, A, B, S, H, hd, W, "bf16", stream)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            tb.pblock_swa_attention(qkv, 3 * A, o, A, B, S, H, hd, W, "bf16", stream)
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    def pairs(B, S, W):
        w = min(W, S)
        return B * H * (S * w - w * (w - 1) // 2)

    points = []
    for S, W in [(8192, w) for w in (128, 256, 512, 1024, 2048)] + [(2048, 1024), (4096, 1024)]:
        ms = time_attention(1, S, W)
        points.append({"B": 1, "S": S, "W": W, "pairs": pairs(1, S, W), "ms": round(ms, 5),
                       "tflops": round(4 * hd * pairs(1, S, W) / (ms * 1e-3) / 1e12, 1)})
        print(f"[sweep] S={S} W={W}: {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    x = np.array([p["pairs"] for p in points], dtype=np.float64)
    y = np.array([p["ms"] for p in points], dtype=np.float64)
    slope, icpt = np.polyfit(x, y, 1)
    r2 = 1.0 - float(((y - (slope * x + icpt)) ** 2).sum() / ((y - y.mean()) ** 2).sum())
    fc = CONFIGS["fullcausal"]
    ms_fc = time_attention(fc.B, fc.S, fc.W)
    pred_fc = slope * pairs(fc.B, fc.S, fc.W) + icpt
    print(json.dumps({
        "sweep": "swa_attention bf16, 32 heads x 128 (the long workload's heads)",
        "points": points,
        "fit": {"ms_per_gpair": round(slope * 1e9, 6), "intercept_ms": round(icpt, 5), "r2": round(r2, 5)},
        "fullcausal_check": {"B": fc.B, "S": fc.S, "W": fc.W, "ms": round(ms_fc, 5), "predicted_ms": round(pred_fc, 5),
                             "ratio": round(ms_fc / pred_fc, 3)},
    }), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the block runs on one GPU's "
              "share at its real shape, and the library has no collectives. Run with --gpus 1.", file=sys.stderr,
              flush=True)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import transformer_block_fwd_amd as tb
    from workload import CONFIGS, make_dy, make_inputs, make_ln2, make_variant_params

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.sweep:
        attention_sweep()
        return
    if args.vs_torch_gemm:
        gemm_vs_torch()
        return

    cfg = CONFIGS[args.workload]
    if args.window:
        cfg = cfg.replace(W=args.window)
    if args.add_residual is not None:
        cfg = cfg.replace(add_residual=args.add_residual)
    if args.block == "serial":
        cfg = cfg.replace(add_residual=1)  # the serial form's residual stream
    print(f"[bench] workload {cfg} block {args.block}", file=sys.stderr, flush=True)
    inp = make_inputs(cfg, seed=0)
    arrs = inp.device_arrays()
    ln2 = make_ln2(cfg, seed=0)
    arrs["gamma2"], arrs["beta2"] = ln2["gamma2_dev"], ln2["beta2_dev"]
    use_variant = bool(args.gelu_tanh or args.bias or args.rope or args.two_ln)
    if use_variant and args.block != "parallel":
        raise SystemExit("the variant switches apply to the parallel block")
    vp = make_variant_params(cfg, seed=0)
    if args.bias:
        arrs["b_in"], arrs["b_out"] = vp["b_in_dev"], vp["b_out_dev"]
    if cfg.dtype == "bf16":
        dev = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).cuda()
               for k, v in arrs.items()}
    else:
        dev = {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda() for k, v in arrs.items()}
    out = torch.empty_like(dev["x"])
    weights = (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"])
    stream = torch.cuda.current_stream()
    h = tb.pblock_create(cfg)

    if args.chunks and (args.block != "parallel" or use_variant):
        raise SystemExit("--chunks applies to the parallel block without variant switches")
    variant = tb.make_variant(gelu_tanh=args.gelu_tanh, rope=bool(args.rope), rope_base=args.rope or 10000.0,
                              two_ln=args.two_ln)
    extra = {k: dev[k] for k in ("b_in", "b_out") if k in dev}
    if args.two_ln:
        extra.update(ln2_gamma=dev["gamma2"], ln2_beta=dev["beta2"])
    variant_desc = None
    oracle_variant = None
    if use_variant:
        variant_desc = {"gelu": "tanh" if args.gelu_tanh else "erf", "bias": bool(args.bias),
                        "rope_base": args.rope or None, "two_ln": bool(args.two_ln)}
        oracle_variant = dict(gelu_form=variant_desc["gelu"], rope_base=variant_desc["rope_base"])
        if args.bias:
            oracle_variant.update(b_in=vp["b_in"], b_out=vp["b_out"])
        if args.two_ln:
            oracle_variant.update(gamma2=ln2["gamma2"], beta2=ln2["beta2"])
    done = [torch.cuda.Event(enable_timing=True) for _ in range(args.chunks)]
    ready = [None] * args.chunks if args.chunk_input else None
    if args.chunk_input and not args.chunks:
        raise SystemExit("--chunk-input needs --chunks")
    if args.rowchunks and (not args.chunks or args.chunk_input or cfg.dtype != "bf16"):
        raise SystemExit("--rowchunks needs --chunks (whole input, bf16)")
    flags = torch.zeros(max(args.chunks, 1), dtype=torch.int32, device="cuda")
    epoch = [0]
    train_dy = None
    if args.train:
        if args.block != "parallel" or use_variant or args.chunks or cfg.dtype != "bf16":
            raise SystemExit("--train times the plain bf16 parallel block")
        dyd = make_dy(cfg, seed=0)
        train_dy = dyd["dy"]
        dy_dev = torch.from_numpy(np.ascontiguousarray(dyd["dy_dev"]).view(np.int16)).view(torch.bfloat16).cuda()
        train_ws = torch.empty(tb.pblock_train_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
        grads = {"dx": torch.empty_like(dev["x"]), "dln_gamma": torch.empty_like(dev["gamma"]),
                 "dln_beta": torch.empty_like(dev["beta"]), "dw_in": torch.empty_like(dev["w_in"]),
                 "dw_out": torch.empty_like(dev["w_out"])}

    if args.ramp:
        def series(n, timing):
            tb.pblock_set_timing(h, timing)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            ev[0].record(stream)
            for i in range(n):
                tb.pblock_forward(h, dev["x"], weights, cfg, out, stream)
                ev[i + 1].record(stream)
            torch.cuda.synchronize()
            tb.pblock_set_timing(h, False)
            return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]

        for _ in range(5):
            tb.pblock_forward(h, dev["x"], weights, cfg, out, stream)
        torch.cuda.synchronize()
        cold_start = series(120, False)
        on1, off, on2 = series(60, True), series(60, False), series(60, True)
        print(json.dumps({
            "ramp": f"{cfg.name} forward from a cold start, 5 warm-up steps, then one event per step",
            "median_ms_per_10_steps": [round(percentile(cold_start[i:i + 10], 0.5), 5) for i in range(0, 120, 10)],
            "per_kernel_events_on_off_on_median_ms": [round(percentile(v, 0.5), 5) for v in (on1, off, on2)],
        }), flush=True)
        tb.pblock_destroy(h)
        return

    def step(chunked=bool(args.chunks)):
        if args.train:
            tb.pblock_forward_train(h, dev["x"], weights, cfg, out, train_ws, stream)
            tb.pblock_backward(h, dev["x"], weights, cfg, dy_dev, grads, train_ws, stream)
        elif args.block == "serial":
            tb.pblock_forward_serial(h, dev["x"], weights, (dev["gamma2"], dev["beta2"]), cfg, out, stream)
        elif use_variant:
            tb.pblock_forward_variant(h, dev["x"], weights, extra, cfg, variant, out, stream)
        elif chunked and args.rowchunks:
            epoch[0] = epoch[0] % 0x7FFFFFFF + 1
            tb.pblock_forward_rowchunks(h, dev["x"], weights, cfg, out, args.chunks, flags, epoch[0], stream)
        elif chunked:
            tb.pblock_forward_chunked(h, dev["x"], weights, cfg, out, args.chunks, ready, done, stream)
        else:
            tb.pblock_forward(h, dev["x"], weights, cfg, out, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    # The timed region: exactly K steps between two events, nothing else recorded in it (per-kernel
    # events would add ~2% to each step).
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = t0.elapsed_time(t1)
    print(f"[bench] timed {args.steps} steps in {ms_total:.3f} ms (wall {wall * 1e3:.3f} ms)", file=sys.stderr,
          flush=True)

    # The same K steps again with HIP events around every step and every kernel launch (the
    # library's per-kernel timing, on the stream the kernels run on): the per-step spread, the
    # per-kernel times and the roofline record come from here.
    tb.pblock_set_timing(h, True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_instrumented = marks[0].elapsed_time(marks[-1])
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    kernel_ms, n_fwd = tb.pblock_kernel_times(h, backward=args.train)
    if args.train:
        n_fwd //= 2  # a forward and a backward call per step
    tb.pblock_set_timing(h, False)

    chunking = None
    published_us = None
    # completion of each chunk's rows of out within the last timed step (before any more steps)
    t_done = [marks[-2].elapsed_time(e) for e in done] if args.chunks and not args.rowchunks else None
    if args.chunks:
        # the chunked and the unchunked forward in alternating rounds of 10 steps (5 rounds each),
        # for a ratio that clock and temperature drift over the run does not bias
        ab = {False: [], True: []}
        for _ in range(5):
            for chunked_round in (False, True):
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record(stream)
                for _ in range(10):
                    step(chunked=chunked_round)
                a1.record(stream)
                torch.cuda.synchronize()
                ab[chunked_round].append(a0.elapsed_time(a1) / 10)
        unchunked, chunked_alt = percentile(ab[False], 0.5), percentile(ab[True], 0.5)
    if args.rowchunks:
        # one more step with the consumer on a second stream: when each chunk's flag was seen
        send = torch.empty_like(out)
        stamps = torch.zeros(args.chunks, dtype=torch.int64, device="cuda")
        from transformer_block_fwd_amd.streams import cu_masked_stream, destroy_stream

        n_cus = torch.cuda.get_device_properties(0).multi_processor_count
        side = cu_masked_stream(n_cus - 32, 32, n_cus)  # a hardware queue of its own, the last 32 CUs
        prod = torch.cuda.Stream()  # not the null stream, which would wait for the consumer
        torch.cuda.synchronize()
        epoch[0] = epoch[0] % 0x7FFFFFFF + 1
        tb.pblock_pack_chunks(out, cfg, args.chunks, flags, epoch[0], send, stamps, side)
        tb.pblock_forward_rowchunks(h, dev["x"], weights, cfg, out, args.chunks, flags, epoch[0], prod)
        torch.cuda.synchronize()
        destroy_stream(side)
        st = [int(v) & 0xFFFFFFFFFFFFFFFF for v in stamps.cpu().tolist()]
        if any(v == 0xFFFFFFFFFFFFFFFF for v in st):
            print("[bench] the consumer timed out waiting for a chunk", file=sys.stderr, flush=True)
        else:
            published_us = [round((v - min(st)) / 100.0, 2) for v in st]  # 100 MHz device clock
            print(f"[bench] chunk publication (us after the first): {published_us}", file=sys.stderr, flush=True)
    if args.chunks:
        # the same forward unchunked, with per-kernel timing, for the kernel and roofline figures
        tb.pblock_set_timing(h, True)
        for _ in range(max(5, args.steps // 3)):
            step(chunked=False)
        torch.cuda.synchronize()
        kernel_ms, n_fwd = tb.pblock_kernel_times(h)
        tb.pblock_set_timing(h, False)
        chunking = {"chunks": args.chunks, "input_chunked": bool(args.chunk_input),
                    "form": "one output-GEMM launch, flags" if args.rowchunks else "one launch per chunk, events",
                    "chunk_done_ms": [round(v, 5) for v in t_done] if t_done else None,
                    "published_us_after_first": published_us,
                    "unchunked_ms_per_step": round(unchunked, 5),
                    "alternating_rounds_ms": {"chunked": round(chunked_alt, 5), "unchunked": round(unchunked, 5)},
                    "chunked_over_unchunked": round(chunked_alt / unchunked, 4)}
        if t_done:
            print(f"[bench] chunk completion (ms into the step): {[round(v, 3) for v in t_done]}", file=sys.stderr,
                  flush=True)

    cold = None
    if args.cold_steps > 0:
        scrub = torch.empty(COLD_SCRUB_MIB << 20, dtype=torch.uint8, device="cuda")
        cold_ms = []
        for i in range(args.cold_steps):
            scrub.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            cold_ms.append(e0.elapsed_time(e1))
        del scrub
        med = percentile(cold_ms, 0.5)
        cold = {"steps": args.cold_steps, "scrub_mib": COLD_SCRUB_MIB, "median_ms": round(med, 5),
                "tflops": round(cfg.flops() / (med * 1e-3) / 1e12, 3)}
        print(f"[bench] cold-cache median {med:.3f} ms", file=sys.stderr, flush=True)

    # a plain device copy of x's bytes (read M*d, write M*d), back to back so x stays in the
    # last-level cache: an upper bound for LayerNorm, which inside the step reads x after the
    # GEMMs have streamed the weights through that cache
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        out.copy_(dev["x"])
    c0.record(stream)
    for _ in range(20):
        out.copy_(dev["x"])
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * dev["x"].numel() * dev["x"].element_size() / (c0.elapsed_time(c1) / 20 * 1e-3) / 1e9

    mfma_tflops = mfma_loop_rate(tb, torch, stream)
    mfma32_tflops = mfma_loop_rate(tb, torch, stream, form="32x32x16")
    print(f"[bench] register-only MFMA loop {mfma_tflops:.1f} TFLOP/s (16x16x32; 32x32x16: {mfma32_tflops:.1f})",
          file=sys.stderr, flush=True)

    ms_step = ms_total / args.steps
    flops = cfg.flops() + (backward_flops(cfg) if args.train else 0.0)
    tflops = flops / (ms_step * 1e-3) / 1e12
    k_avg = {k: v / max(n_fwd, 1) for k, v in kernel_ms.items()}
    g1_ms = k_avg["gemm_in"]
    g1_flops = cfg.gemm1_flops()
    as_profiled = (args.block == "parallel" and not args.window and args.add_residual is None and not args.chunks
                   and not use_variant and not args.train)
    traffic = MEASURED_TRAFFIC_BYTES.get(cfg.name) if as_profiled else None
    roofline = {"kernel": "gemm_in (fused QKV+FC1 GEMM, GeLU epilogue)", "bound": "mfma",
                "achieved": round(g1_flops / (g1_ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g1_flops / (g1_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flops_per_launch": g1_flops, "avg_launch_ms": round(g1_ms, 5)}
    if args.block == "serial" or args.two_ln:
        roofline["kernel"] = "gemm_in (QKV GEMM + FC1 GEMM with GeLU epilogue, summed per forward)"
    per_kernel = {}
    for k, ms in k_avg.items():
        kf = {"gemm_in": cfg.gemm1_flops(), "gemm_out": cfg.gemm2_flops(), "attention": cfg.attn_flops(),
              "bwd_gemm_dgrad": cfg.gemm1_flops() + cfg.gemm2_flops(),
              "bwd_gemm_wgrad": cfg.gemm1_flops() + cfg.gemm2_flops(),
              "bwd_attention": 2.5 * cfg.attn_flops()}.get(k)
        rec = {"ms": round(ms, 5)}
        if kf:
            rec["tflops"] = round(kf / (ms * 1e-3) / 1e12, 2)
        if k == "layernorm":
            es = 2 if cfg.dtype == "bf16" else 4
            n_ln = 2 if (args.block == "serial" or args.two_ln) else 1
            rec["gbs"] = round(n_ln * (2 * cfg.M * cfg.d * es + 2 * cfg.d * es) / (ms * 1e-3) / 1e9, 1)
            rec["plain_copy_warm_gbs"] = round(copy_gbs, 1)
        per_kernel[k] = rec

    result = {
        "metric": METRIC if not args.train else METRIC_TRAIN,
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
        "config": {"workload": f"{cfg.name}: {WORKLOAD_NOTES.get(cfg.name, '')}", "block": args.block, "B": cfg.B,
                   "S": cfg.S, "d": cfg.d, "H": cfg.H, "hd": cfg.hd, "ffn": cfg.ffn, "W": cfg.W,
                   "add_residual": cfg.add_residual, "parallelism": "single GPU", "variant": variant_desc,
                   "step": "forward + backward" if args.train else "forward"},
        "pct_peak_bf16": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(cfg.M / (ms_step * 1e-3), 1),
        "algorithmic_gflop_per_step": round(flops / 1e9, 3),
        # the instrumented pass of the same K steps (events around every step and kernel launch)
        "instrumented": {"ms_per_step": round(ms_instrumented / args.steps, 5),
                         "step_ms": {"median": round(percentile(step_ms, 0.5), 5),
                                     "p10": round(percentile(step_ms, 0.1), 5),
                                     "p90": round(percentile(step_ms, 0.9), 5)}},
        "cold_cache": cold,
        "chunking": chunking,
        "mfma_loop_tflops": round(mfma_tflops, 1),
        "mfma_loop_32x32x16_tflops": round(mfma32_tflops, 1),
        "pct_of_mfma_loop": round(100 * tflops / mfma_tflops, 2),
        "kernels": per_kernel,
        "roofline": roofline,
    }
    tb.pblock_destroy(h)
    del dev, out
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.block, ln2, oracle_variant, train_dy)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
