"""Benchmark: Q8_0 decode-layer GEMV set on one MI355X.

One step is one pass of a 3B-class decode layer's weight-streaming products at
batch 1, all in libqdec kernels on one stream:
    fused QKV   Wq 3072x3072, Wk/Wv 1024x3072 (GQA), one shared x[3072]
    FFN up      8192x3072, x[3072]
    FFN down    3072x8192 with residual, x[8192], r[3072]
Weights are seeded synthetic Q8_0 (W ~ N(0, 0.02) quantised per 32-block),
activations N(0, 1).  Consecutive steps read the weights of consecutive
"layers": LAYERS distinct device copies (8 x 70 MB = 560 MB, twice the 256 MB
Infinity Cache), so the bytes come from HBM as in a real decode.

value = algorithmic bytes per step (GGML weight bytes + x + out + residual)
        / wall time per step, in GB/s, inputs resident in HBM.
roofline = the dominant kernel's algorithmic bytes per launch / its mean
        launch duration from HIP events recorded around each of its launches
        inside the timed steps, against 8 TB/s.
cpu_baseline = the CPU oracle (single thread) on a bounded sample of steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
LAYERS = 8
N_IN, N_Q, N_KV, N_FF = 3072, 3072, 1024, 8192


def q8_bytes(n_out, n_in):
    return n_out * (n_in // 32) * 34


def step_bytes():
    qkv = q8_bytes(N_Q + 2 * N_KV, N_IN) + N_IN * 4 + (N_Q + 2 * N_KV) * 4
    up = q8_bytes(N_FF, N_IN) + N_IN * 4 + N_FF * 4
    down = q8_bytes(N_IN, N_FF) + N_FF * 4 + N_IN * 4 * 2
    return {"qkv": qkv, "up": up, "down_residual": down}


def make_inputs():
    import synth
    cfg = 1
    w = {
        "wq": synth.q8_0_weights(synth.seed(cfg, 0), N_Q, N_IN)[0],
        "wk": synth.q8_0_weights(synth.seed(cfg, 1), N_KV, N_IN)[0],
        "wv": synth.q8_0_weights(synth.seed(cfg, 2), N_KV, N_IN)[0],
        "up": synth.q8_0_weights(synth.seed(cfg, 3), N_FF, N_IN)[0],
        "down": synth.q8_0_weights(synth.seed(cfg, 4), N_IN, N_FF)[0],
    }
    x = {
        "x_qkv": synth.normal_f32(synth.seed(cfg, 5), (1, N_IN)),
        "x_up": synth.normal_f32(synth.seed(cfg, 6), (1, N_IN)),
        "x_down": synth.normal_f32(synth.seed(cfg, 7), (1, N_FF)),
        "r_down": synth.normal_f32(synth.seed(cfg, 8), (1, N_IN)),
    }
    return w, x


def cpu_baseline(w, x, budget_s=12.0):
    """The oracle as it stands, one thread, timed on whole steps until the
    budget is spent (at least one step)."""
    import oracle
    steps, t0 = 0, time.perf_counter()
    while True:
        oracle.q8_0_qkv(w["wq"], w["wk"], w["wv"], N_IN, N_Q, N_KV, x["x_qkv"])
        oracle.q8_0_gemv(w["up"], N_IN, N_FF, x["x_up"])
        oracle.q8_0_gemv_residual(w["down"], N_FF, N_IN, x["x_down"], x["r_down"])
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            break
    total = sum(step_bytes().values())
    return {"value": round(total * steps / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full decode-layer steps (QKV + up + down/residual, batch 1) in {dt:.1f} s, "
                      f"single-threaded C oracle, f64 accumulation"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is a "
              "single-GPU weight-streaming kernel and no multi-GPU build exists", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_decode_ggml_amd as qd

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    w_host, x_host = make_inputs()
    print(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    # LAYERS device copies of every weight, repacked once (load time, untimed)
    layers = []
    base = {k: torch.from_numpy(v).to(dev) for k, v in w_host.items()}
    for _ in range(LAYERS):
        L = {k: v.clone() for k, v in base.items()}
        qd.prepare(L["wq"], qd.TYPE_Q8_0, N_IN, N_Q)
        qd.prepare(L["wk"], qd.TYPE_Q8_0, N_IN, N_KV)
        qd.prepare(L["wv"], qd.TYPE_Q8_0, N_IN, N_KV)
        qd.prepare(L["up"], qd.TYPE_Q8_0, N_IN, N_FF)
        qd.prepare(L["down"], qd.TYPE_Q8_0, N_FF, N_IN)
        layers.append(L)
    del base
    xs = {k: torch.from_numpy(v).to(dev) for k, v in x_host.items()}
    q_out = torch.empty((1, N_Q), device=dev)
    k_out = torch.empty((1, N_KV), device=dev)
    v_out = torch.empty((1, N_KV), device=dev)
    up_out = torch.empty((1, N_FF), device=dev)
    down_out = torch.empty((1, N_IN), device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    names = ("qkv", "up", "down_residual")
    events = {n: [] for n in names}

    def step(i, record):
        L = layers[i % LAYERS]
        calls = (
            ("qkv", lambda: qd.q8_0_qkv(L["wq"], L["wk"], L["wv"], N_IN, N_Q, N_KV, xs["x_qkv"],
                                        q_out, k_out, v_out, stream=stream)),
            ("up", lambda: qd.q8_0_gemv(L["up"], N_IN, N_FF, xs["x_up"], out=up_out, stream=stream)),
            ("down_residual", lambda: qd.q8_0_gemv_residual(L["down"], N_FF, N_IN, xs["x_down"],
                                                            xs["r_down"], out=down_out, stream=stream)),
        )
        for name, fn in calls:
            if record:
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record(stream)
                fn()
                e.record(stream)
                events[name].append((s, e))
            else:
                fn()

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()

    # One HIP graph per layer (its three launches), captured on torch's capture
    # stream, plus one graph over all LAYERS layers; replaying them removes the
    # per-call Python/ctypes cost from the device timeline.
    graphs = []
    for i in range(LAYERS):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            stream = torch.cuda.current_stream()
            step(i, False)
        graphs.append(g)
    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all):
        stream = torch.cuda.current_stream()
        for i in range(LAYERS):
            step(i, False)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        g_all.replay()
    torch.cuda.synchronize()

    # timed region 1: exactly args.steps steps through the graphs (headline)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    full, rest = divmod(args.steps, LAYERS)
    for _ in range(full):
        g_all.replay()
    for i in range(rest):
        graphs[i].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # eager steps (one host call per product), for reference
    launches0 = qd.launch_count()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, False)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    assert qd.launch_count() - launches0 == 3 * args.steps, "not every product ran in libqdec"

    # timed region 2: the same steps with HIP events around every launch
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    per_kernel = {}
    sb = step_bytes()
    for n in names:
        us = np.array([s.elapsed_time(e) * 1e3 for s, e in events[n]])
        per_kernel[n] = {"mean_us": round(float(us.mean()), 3), "median_us": round(float(np.median(us)), 3),
                         "bytes": sb[n], "gbs": round(sb[n] / (us.mean() * 1e-6) / 1e9, 1)}
    dom = max(names, key=lambda n: per_kernel[n]["mean_us"])
    achieved = per_kernel[dom]["gbs"]

    total_bytes = sum(sb.values())
    ms_per_step = wall / args.steps * 1e3
    value = total_bytes / (wall / args.steps) / 1e9

    line = {
        "metric": "Q8_0 decode GEMV achieved HBM GB/s (% of peak); batched GEMM TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Q8_0 decode layer GEMV set, batch 1: fused QKV (n_q 3072, n_kv 1024, n_in 3072) "
                        "+ FFN up 8192x3072 + FFN down 3072x8192 with residual",
            "batch": 1,
            "layers_rotated": LAYERS,
            "bytes_per_step": total_bytes,
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "kernels": per_kernel,
            "launch": "hip graph per layer (3 kernels), replayed",
            "eager_ms_per_step": round(wall_eager / args.steps * 1e3, 5),
        },
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w_host, x_host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
