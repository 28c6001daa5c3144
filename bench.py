"""Benchmark: Q8_0 decode-layer GEMV set on one MI355X.

One step is one pass of a 3B-class decode layer's weight-streaming products at
batch 1, all in libqdec kernels on one stream:
    fused QKV   Wq 3072x3072, Wk/Wv 1024x3072 (GQA), one shared x[3072]
    FFN up      8192x3072, x[3072]
    FFN down    3072x8192 with residual, x[8192], r[3072]
Weights are seeded synthetic Q8_0 (W ~ N(0, 0.02) quantised per 32-block),
activations N(0, 1).  Consecutive steps read the weights of consecutive
"layers": LAYERS distinct device copies (32 x 70 MB = 2.25 GB; even one product
alone rotates over >= 512 MB, twice the 256 MB Infinity Cache), so the bytes
come from HBM as in a real decode.

value = algorithmic bytes per step (GGML weight bytes + x + out + residual)
        / wall time per step, in GB/s, inputs resident in HBM.  The timed
        region is one replay of a HIP graph that holds exactly `steps` steps
        (3 launches each, layers rotating), bracketed by device syncs.
roofline = the dominant kernel's algorithmic bytes per launch / its mean
        launch duration (HIP events around a replayed graph of `steps`
        launches of that kernel), against 8 TB/s; traffic = the HBM bytes the
        profiler counted for one launch of it (profiles/, null once the GEMV
        sources differ from the ones profiled).
batched_gemm = the prefill-shaped Q8_0 GEMM (batch 128 and 512 rows against
        the layers' FFN up and down weights, the other half of the metric):
        mean launch duration of graph-replayed launches, TFLOP/s and the
        fraction of the 2.5 PFLOP/s dense bf16 matrix-core peak.
cpu_baseline = the CPU oracle on a bounded sample of steps, single-threaded
        and on all host cores (row slices of every product in a thread pool).
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
BF16_PEAK_TFLOPS = 2500.0
LAYERS = 32
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


def measured_traffic(kernel_role):
    """HBM bytes per launch of one decode-layer kernel, as counted by the
    profiler (profiles/q8_0_decode_layer_traffic.json), or None when the
    kernel sources changed after the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "q8_0_decode_layer_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        for rel, digest in rec["source_sha256"].items():
            with open(os.path.join(ROOT, rel), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None, None
        k = rec["kernels"][kernel_role]
    except (OSError, KeyError, ValueError):
        return None, None
    return k["hbm_bytes"], {"fetch_KiB": k["FETCH_SIZE_KiB"], "write_KiB": k["WRITE_SIZE_KiB"],
                            "fetch_scale": rec["calibration"]["fetch_scale"],
                            "write_scale": rec["calibration"]["write_scale"],
                            "algorithmic_bytes": k["algorithmic_bytes"],
                            "source": "profiles/q8_0_decode_layer_traffic.json"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores():
    """Worker threads for the all-core baseline: the CPUs this process may
    run on, at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_step_single(w, x):
    import oracle
    oracle.q8_0_qkv(w["wq"], w["wk"], w["wv"], N_IN, N_Q, N_KV, x["x_qkv"])
    oracle.q8_0_gemv(w["up"], N_IN, N_FF, x["x_up"])
    oracle.q8_0_gemv_residual(w["down"], N_FF, N_IN, x["x_down"], x["r_down"])


def cpu_step_tasks(w, x, parts):
    """The step as independent row-slice calls of the unchanged oracle: every
    product's output rows split into `parts` contiguous slices (the fused QKV
    is its three products, as the oracle defines it)."""
    import oracle
    tasks = []

    def slices(n_out):
        edges = [n_out * k // parts for k in range(parts + 1)]
        return [(a, b) for a, b in zip(edges[:-1], edges[1:]) if b > a]

    for key, n_in, n_out, xk in (("wq", N_IN, N_Q, "x_qkv"), ("wk", N_IN, N_KV, "x_qkv"),
                                 ("wv", N_IN, N_KV, "x_qkv"), ("up", N_IN, N_FF, "x_up")):
        rb = (n_in // 32) * 34
        for a, b in slices(n_out):
            tasks.append(lambda key=key, n_in=n_in, xk=xk, a=a, b=b, rb=rb:
                         oracle.q8_0_gemv(w[key][a * rb:b * rb], n_in, b - a, x[xk]))
    rb = (N_FF // 32) * 34
    for a, b in slices(N_IN):
        tasks.append(lambda a=a, b=b: oracle.q8_0_gemv_residual(w["down"][a * rb:b * rb], N_FF, b - a,
                                                                x["x_down"], x["r_down"][:, a:b]))
    return tasks


def cpu_baseline(w, x, budget_s=12.0):
    """The oracle as it stands, timed on whole steps until each budget is
    spent (at least one step): one thread, then all host cores (the C oracle
    releases the GIL, so a thread pool runs its row slices in parallel)."""
    import concurrent.futures as cf
    total = sum(step_bytes().values())
    steps, t0 = 0, time.perf_counter()
    while True:
        cpu_step_single(w, x)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            break
    single = {"value": round(total * steps / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
              "sample": f"{steps} full decode-layer steps (QKV + up + down/residual, batch 1) in {dt:.1f} s, "
                        f"single-threaded C oracle, f64 accumulation"}
    n = host_cores()
    tasks = cpu_step_tasks(w, x, 4 * n)
    steps, t0 = 0, time.perf_counter()
    with cf.ThreadPoolExecutor(n) as ex:
        while True:
            for f in [ex.submit(t) for t in tasks]:
                f.result()
            steps += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s:
                break
    allc = {"value": round(total * steps / dt / 1e9, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"{steps} full decode-layer steps in {dt:.1f} s, the unchanged C oracle on {len(tasks)} "
                      f"row slices per step in a pool of {n} threads"}
    allc["cpu_model"] = single["cpu_model"] = cpu_model()
    return allc, single


def fingerprints(w, x):
    """FNV-1a fingerprint of every input tensor (the pages' weight_fingerprint
    key), printed to the run log so that runs can be audited."""
    import synth
    dims = {"wq": (N_IN, N_Q), "wk": (N_IN, N_KV), "wv": (N_IN, N_KV), "up": (N_IN, N_FF), "down": (N_FF, N_IN),
            "x_qkv": (N_IN, 1), "x_up": (N_IN, 1), "x_down": (N_FF, 1), "r_down": (N_IN, 1)}
    out = {}
    for k, v in list(w.items()) + list(x.items()):
        n_in, n_out = dims[k]
        out[k] = f"{synth.fnv1a64(v, n_in, n_out):016x}"
    return out


def ceiling(args):
    """The plain streaming-read ceiling (qdec_stream_read) at the byte counts
    of the decode products: one JSON line per (size, loads per lane), mean
    launch duration of graph-replayed launches over rotated regions of a
    2.5 GB buffer (>= 512 MB per size, twice the Infinity Cache)."""
    import torch

    import quantized_decode_ggml_amd as qd
    dev = torch.device("cuda:0")
    total = 2560 << 20
    buf = torch.randint(0, 256, (total,), dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    sizes = (("QKV 5120x3072 Q8_0", q8_bytes(5120, 3072)), ("FFN 8192x3072 Q8_0", q8_bytes(8192, 3072)),
             ("Q4_K 8192x3072", 8192 * 12 * 144), ("vocab 128256x3072 Q8_0", q8_bytes(128256, 3072)))
    for name, nbytes in sizes:
        nbytes -= nbytes % 16
        stride = -(-nbytes // 4096) * 4096
        regions = max(2, min(total // stride, -(-(512 << 20) // nbytes)))
        for u in (1, 2, 4, 8, 16):
            offs = [r * stride for r in range(regions)]
            iters = 40 if nbytes > (100 << 20) else 200
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for i in range(2 * regions):
                    qd.stream_read(buf[offs[i % regions]:], nbytes, u, sink)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(iters):
                    qd.stream_read(buf[offs[i % regions]:], nbytes, u, sink)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            cur = torch.cuda.current_stream()
            e0.record(cur)
            g.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / iters
            print(json.dumps({"ceiling": name, "bytes": nbytes, "loads_per_lane": u, "mean_us": round(us, 3),
                              "gbs": round(nbytes / us / 1e3, 1),
                              "pct_hbm": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 2)}), flush=True)
            del g


def calibration_copy(qd, torch, dev):
    """64 MiB read + 64 MiB written by qdec_copy_kernel, three times: the
    known-size reference that scales the profiler's HBM byte counters."""
    nbytes = 64 << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        qd.copy(dst, src, nbytes)
    torch.cuda.synchronize()
    del src, dst


def suite(args):
    """Every workload configuration through the library, one line of JSON each
    (to stdout): mean launch duration of graph-replayed launches on rotated
    weight copies (>= 512 MB per workload), GB/s of algorithmic bytes and, for
    the batched GEMMs, TFLOP/s."""
    import numpy as np
    import torch

    import quantized_decode_ggml_amd as qd
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.calibrate:
        calibration_copy(qd, torch, dev)

    def copies_for(nbytes):
        return max(2, -(-(512 << 20) // max(nbytes, 1)))

    def timed(name, launches, nbytes, flops=None, iters=100, warm=20, extra=None):
        """Mean launch duration: `iters` launches (rotating over the weight
        copies) captured into one HIP graph, replayed, bracketed by HIP events
        on the replay stream; host launch costs stay out of the device timeline.
        Warm-up and capture use one dedicated stream, so per-stream library
        state (the batched GEMV workspace) exists before the capture starts."""
        nonlocal stream
        if args.only and not name.startswith(args.only):
            return                      # --only: this line is not wanted (its inputs were still made)
        n = len(launches)
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            for i in range(warm):
                launches[i % n]()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            stream = torch.cuda.current_stream()
            for i in range(iters):
                launches[i % n]()
        stream = torch.cuda.current_stream()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del g
        us = e0.elapsed_time(e1) * 1e3 / iters
        rec = {"workload": name, "mean_us": round(us, 3), "bytes": int(nbytes),
               "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
               "pct_hbm": round(100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        if flops:
            rec["tflops"] = round(flops / (us * 1e-6) / 1e12, 2)
        if extra:
            rec.update(extra)
        print(json.dumps(rec), flush=True)

    def q8_dev(cfg, idx, n_out, n_in, ncopies):
        raw = torch.from_numpy(synth.q8_0_weights(synth.seed(cfg, idx), n_out, n_in)[0]).to(dev)
        out = []
        for _ in range(ncopies):
            c = raw.clone()
            qd.prepare(c, qd.TYPE_Q8_0, n_in, n_out)
            out.append(c)
        return out

    def xdev(seed, shape):
        return torch.from_numpy(synth.normal_f32(seed, shape)).to(dev)

    # config 0
    w0 = q8_dev(0, 0, 256, 512, 4)
    x0, o0 = xdev(synth.seed(0, 1), (1, 512)), torch.empty((1, 256), device=dev)
    timed("c0 q8_0_gemv 256x512 b1", [lambda w=w: qd.q8_0_gemv(w, 512, 256, x0, out=o0) for w in w0],
          q8_bytes(256, 512) + 512 * 4 + 256 * 4)
    # config 1
    nqkv = q8_bytes(5120, 3072)
    L = copies_for(nqkv)
    wq, wk, wv = q8_dev(1, 0, 3072, 3072, L), q8_dev(1, 1, 1024, 3072, L), q8_dev(1, 2, 1024, 3072, L)
    xq = xdev(synth.seed(1, 5), (1, 3072))
    oq, ok, ov = (torch.empty((1, n), device=dev) for n in (3072, 1024, 1024))
    timed("c1 q8_0_qkv 3072+1024+1024 x 3072 b1",
          [lambda i=i: qd.q8_0_qkv(wq[i], wk[i], wv[i], 3072, 3072, 1024, xq, oq, ok, ov) for i in range(L)],
          nqkv + 3072 * 4 + 5120 * 4)
    del wq, wk, wv
    L = copies_for(q8_bytes(8192, 3072))
    wup = q8_dev(1, 3, 8192, 3072, L)
    xu, ou = xdev(synth.seed(1, 6), (1, 3072)), torch.empty((1, 8192), device=dev)
    timed("c1 q8_0_gemv up 8192x3072 b1", [lambda w=w: qd.q8_0_gemv(w, 3072, 8192, xu, out=ou) for w in wup],
          q8_bytes(8192, 3072) + 3072 * 4 + 8192 * 4)
    wdn = q8_dev(1, 4, 3072, 8192, L)
    xd, rd, od = xdev(synth.seed(1, 7), (1, 8192)), xdev(synth.seed(1, 8), (1, 3072)), torch.empty((1, 3072), device=dev)
    timed("c1 q8_0_gemv_residual down 3072x8192 b1",
          [lambda w=w: qd.q8_0_gemv_residual(w, 8192, 3072, xd, rd, out=od) for w in wdn],
          q8_bytes(3072, 8192) + 8192 * 4 + 3072 * 8)
    # config 2 (gate/up rotate in pairs; down reuses the config-1 rotation)
    Lg = copies_for(2 * q8_bytes(8192, 3072))
    wg = q8_dev(2, 0, 8192, 3072, Lg)
    wu2 = q8_dev(2, 1, 8192, 3072, Lg)
    for b in (1, 2, 4, 8):
        x2, m2 = xdev(synth.seed(2, 3) + b, (b, 3072)), torch.empty((b, 8192), device=dev)
        timed(f"c2 q8_0_swiglu 2x8192x3072 b{b}",
              [lambda i=i: qd.q8_0_swiglu(wg[i], wu2[i], 3072, 8192, x2, out=m2) for i in range(Lg)],
              2 * q8_bytes(8192, 3072) + b * 3072 * 4 + b * 8192 * 4)
        r2, o2 = xdev(synth.seed(2, 4) + b, (b, 3072)), torch.empty((b, 3072), device=dev)
        timed(f"c2 q8_0_gemv_residual down 3072x8192 b{b}",
              [lambda w=w: qd.q8_0_gemv_residual(w, 8192, 3072, m2, r2, out=o2) for w in wdn],
              q8_bytes(3072, 8192) + b * 8192 * 4 + b * 3072 * 8)
        # the whole FFN block as one chain: one upload of x from pinned host
        # memory, SwiGLU, down with x as the residual, one readback (the
        # block-level call of the pages); PCIe-inclusive, bytes = weights + x + out
        hx = torch.from_numpy(synth.normal_f32(synth.seed(2, 5) + b, (b, 3072))).pin_memory()
        ho = torch.empty((b, 3072), pin_memory=True)
        xb, mb, ob = torch.empty((b, 3072), device=dev), torch.empty((b, 8192), device=dev), \
            torch.empty((b, 3072), device=dev)

        def ffn_chain(i, xb=xb, mb=mb, ob=ob, hx=hx, ho=ho):
            xb.copy_(hx, non_blocking=True)
            qd.q8_0_swiglu(wg[i % Lg], wu2[i % Lg], 3072, 8192, xb, out=mb)
            qd.q8_0_gemv_residual(wdn[i % len(wdn)], 8192, 3072, mb, xb, out=ob)
            ho.copy_(ob, non_blocking=True)

        timed(f"c2 FFN block b{b}: x upload, SwiGLU, down+residual, readback (4 steps)",
              [lambda i=i: ffn_chain(i) for i in range(max(Lg, len(wdn)))],
              2 * q8_bytes(8192, 3072) + q8_bytes(3072, 8192) + b * 3072 * 8)
    del wg, wu2
    # chained pre-norm block at batch 1 (next-row f2): RMSNorm+QKV, O-proj+residual,
    # RMSNorm+SwiGLU, down+residual; 4 launches per block, blocks rotate
    E, NQ, NKV, FF = 3072, 3072, 1024, 8192
    blk = q8_bytes(NQ + 2 * NKV, E) + q8_bytes(E, NQ) + 2 * q8_bytes(FF, E) + q8_bytes(E, FF)
    Lb = copies_for(blk)
    bw = {k: q8_dev(5, i, r, c, Lb) for i, (k, r, c) in enumerate(
        (("q", NQ, E), ("k", NKV, E), ("v", NKV, E), ("o", E, NQ), ("g", FF, E), ("u", FF, E), ("d", E, FF)))}
    g1 = torch.from_numpy((1.0 + 0.1 * synth.normal_f32(synth.seed(5, 10), (E,))).astype(np.float32)).to(dev)
    g2 = torch.from_numpy((1.0 + 0.1 * synth.normal_f32(synth.seed(5, 11), (E,))).astype(np.float32)).to(dev)
    hb = xdev(synth.seed(5, 12), (1, E))
    qb, kb, vb = (torch.empty((1, n), device=dev) for n in (NQ, NKV, NKV))
    sb = torch.empty((1, FF + E), device=dev)

    def block(i):
        qd.q8_0_rmsnorm_qkv(bw["q"][i], bw["k"][i], bw["v"][i], E, NQ, NKV, hb, g1, 1e-5, q_out=qb, k_out=kb,
                            v_out=vb)
        qd.q8_0_attn_out_ffn(bw["o"][i], bw["g"][i], bw["u"][i], bw["d"][i], E, NQ, FF, hb, qb, g2, 1e-5,
                             scratch=sb)

    # bytes: weights + activations read and written by the four products and the folded norms
    act = 4 * (E + E + (NQ + 2 * NKV) + NQ + 2 * E + E + FF + FF + 2 * E)
    timed("f2 pre-norm block b1 (norm+QKV, O+res, norm+SwiGLU, down+res; 4 launches)",
          [lambda i=i: block(i) for i in range(Lb)], blk + act, iters=40)
    # decode attention (next-row f4): 24 query heads, 8 kv heads, d = 128, f32 cache
    NH, NKV_H, HD = 24, 8, 128
    for n_ctx in (1024, 4096, 8192):
        cache_b = 2 * NKV_H * n_ctx * HD * 4
        Lc = copies_for(cache_b)
        caches = [(xdev(synth.seed(7, 2 * i), (NKV_H, n_ctx, HD)), xdev(synth.seed(7, 2 * i + 1), (NKV_H, n_ctx, HD)))
                  for i in range(Lc)]
        qa = xdev(synth.seed(7, 99), (NH, HD))
        oa = torch.empty((NH, HD), device=dev)
        timed(f"f4 attention decode n_ctx={n_ctx} (24 q / 8 kv heads, d 128, f32 cache)",
              [lambda kc=kc, vc=vc: qd.attention_decode(qa, kc, vc, n_ctx, HD ** -0.5, out=oa) for kc, vc in caches],
              cache_b + 2 * NH * HD * 4, iters=100)
        del caches
    # the whole pre-norm block with real attention at n_ctx 4096: norm+QKV, RoPE+append,
    # attention, O+res, norm+SwiGLU, down+res (7 launches), blocks rotate
    n_ctx = 4096
    kcs = [xdev(synth.seed(8, 2 * i), (NKV_H, n_ctx, HD)) for i in range(Lb)]
    vcs = [xdev(synth.seed(8, 2 * i + 1), (NKV_H, n_ctx, HD)) for i in range(Lb)]
    att = torch.empty((1, NQ), device=dev)

    def full_block(i):
        qd.q8_0_rmsnorm_qkv(bw["q"][i], bw["k"][i], bw["v"][i], E, NQ, NKV, hb, g1, 1e-5, q_out=qb, k_out=kb,
                            v_out=vb)
        qd.rope_kv_append(qb.view(NH, HD), kb.view(NKV_H, HD), vb.view(NKV_H, HD), n_ctx - 1, 500000.0, kcs[i],
                          vcs[i])
        qd.attention_decode(qb.view(NH, HD), kcs[i], vcs[i], n_ctx, HD ** -0.5, out=att.view(NH, HD))
        qd.q8_0_attn_out_ffn(bw["o"][i], bw["g"][i], bw["u"][i], bw["d"][i], E, NQ, FF, hb, att, g2, 1e-5,
                             scratch=sb)

    timed("f4 pre-norm block b1 with attention, n_ctx 4096 (7 launches)", [lambda i=i: full_block(i) for i in range(Lb)],
          blk + act + 2 * NKV_H * n_ctx * HD * 4, iters=40)
    del bw, kcs, vcs
    # config 3: batched GEMM (Q8_0 weights reuse up/down rotations; dense f32 separate)
    for B in (128, 512):
        for nm, ws, n_out, n_in in (("up 8192x3072", wup, 8192, 3072), ("down 3072x8192", wdn, 3072, 8192)):
            x3, o3 = xdev(synth.seed(3, 2) + B, (B, n_in)), torch.empty((B, n_out), device=dev)
            timed(f"c3 q8_0_gemm_batched {nm} B{B}",
                  [lambda w=w: qd.q8_0_gemm_batched(w, n_in, n_out, x3, out=o3) for w in ws],
                  q8_bytes(n_out, n_in) + B * n_in * 4 + B * n_out * 4, flops=2.0 * B * n_out * n_in)
    del wup, wdn
    for nm, n_out, n_in in (("up 8192x3072", 8192, 3072), ("down 3072x8192", 3072, 8192)):
        wf = torch.from_numpy(synth.normal_f32(synth.seed(3, 10), (n_out, n_in), 0.02)).to(dev)
        wfs = [wf] + [wf.clone() for _ in range(copies_for(wf.numel() * 4) - 1)]
        for B in (128, 512):
            x3, o3 = xdev(synth.seed(3, 12) + B, (B, n_in)), torch.empty((B, n_out), device=dev)
            timed(f"c3 f32_gemm_batched {nm} B{B}",
                  [lambda w=w: qd.f32_gemm_batched(w, n_in, n_out, x3, out=o3) for w in wfs],
                  n_out * n_in * 4 + B * n_in * 4 + B * n_out * 4, flops=2.0 * B * n_out * n_in)
        # the same weights with their bf16 copies (qdec_prepare): 2 bytes a weight read
        for w in wfs:
            qd.prepare(w, qd.TYPE_F32, n_in, n_out)
        for B in (128, 512):
            x3, o3 = xdev(synth.seed(3, 12) + B, (B, n_in)), torch.empty((B, n_out), device=dev)
            timed(f"c3 f32_gemm_batched bf16 copy {nm} B{B}",
                  [lambda w=w: qd.f32_gemm_batched(w, n_in, n_out, x3, out=o3) for w in wfs],
                  n_out * n_in * 2 + B * n_in * 4 + B * n_out * 4, flops=2.0 * B * n_out * n_in)
        for w in wfs:
            qd.release(w)
        del wfs, wf
    # config 4
    for n_out, n_in in ((8192, 3072), (3072, 8192)):
        raw = torch.from_numpy(synth.q4k_weights(synth.seed(4, 0 if n_out == 8192 else 1), n_out, n_in)).to(dev)
        nb4 = n_out * (n_in // 256) * 144
        ws = []
        for _ in range(copies_for(nb4)):
            c = raw.clone()
            qd.prepare(c, qd.TYPE_Q4_K, n_in, n_out)
            ws.append(c)
        x4, o4 = xdev(synth.seed(4, 2), (1, n_in)), torch.empty((1, n_out), device=dev)
        timed(f"c4 q4k_gemv {n_out}x{n_in} b1", [lambda w=w: qd.q4k_gemv(w, n_in, n_out, x4, out=o4) for w in ws],
              nb4 + n_in * 4 + n_out * 4)
        for bt in (2, 4, 8):   # several batch rows: the integer matrix-core kernel
            xb, ob = xdev(synth.seed(4, 10 + bt), (bt, n_in)), torch.empty((bt, n_out), device=dev)
            timed(f"c4 q4k_gemv {n_out}x{n_in} b{bt}",
                  [lambda w=w, xb=xb, ob=ob: qd.q4k_gemv(w, n_in, n_out, xb, out=ob) for w in ws],
                  nb4 + bt * (n_in + n_out) * 4)
        del ws, raw
    # Q6_K (next-row f3): the FFN shapes and the output-projection shape
    for n_out, n_in in ((8192, 3072), (3072, 8192), (128256, 3072)):
        raw = torch.from_numpy(synth.q6k_weights(synth.seed(6, n_out % 97), n_out, n_in)).to(dev)
        nb6 = n_out * (n_in // 256) * 210
        ws = []
        for _ in range(copies_for(nb6)):
            c = raw.clone()
            qd.prepare(c, qd.TYPE_Q6_K, n_in, n_out)
            ws.append(c)
        x6, o6 = xdev(synth.seed(6, 50), (1, n_in)), torch.empty((1, n_out), device=dev)
        timed(f"f3 q6k_gemv {n_out}x{n_in} b1", [lambda w=w: qd.q6k_gemv(w, n_in, n_out, x6, out=o6) for w in ws],
              nb6 + n_in * 4 + n_out * 4, iters=40 if n_out > 100000 else 100)
        for bt in (2, 4, 8):
            xb, ob = xdev(synth.seed(6, 60 + bt), (bt, n_in)), torch.empty((bt, n_out), device=dev)
            timed(f"f3 q6k_gemv {n_out}x{n_in} b{bt}",
                  [lambda w=w, xb=xb, ob=ob: qd.q6k_gemv(w, n_in, n_out, xb, out=ob) for w in ws],
                  nb6 + bt * (n_in + n_out) * 4, iters=40 if n_out > 100000 else 100)
        del ws, raw
    wvoc = q8_dev(4, 3, 128256, 3072, 2)
    xv, ov = xdev(synth.seed(4, 4), (1, 3072)), torch.empty((1, 128256), device=dev)
    timed("c4 q8_0_gemv vocab 128256x3072 b1", [lambda w=w: qd.q8_0_gemv(w, 3072, 128256, xv, out=ov) for w in wvoc],
          q8_bytes(128256, 3072) + 3072 * 4 + 128256 * 4, iters=40)
    for bt in (4, 8):   # a batched decode step's output projection (integer matrix-core kernel)
        xb, ob = xdev(synth.seed(4, 20 + bt), (bt, 3072)), torch.empty((bt, 128256), device=dev)
        timed(f"c4 q8_0_gemv vocab 128256x3072 b{bt}",
              [lambda w=w, xb=xb, ob=ob: qd.q8_0_gemv(w, 3072, 128256, xb, out=ob) for w in wvoc],
              q8_bytes(128256, 3072) + bt * (3072 + 128256) * 4, iters=40)
        del xb, ob
    # the same projection with the on-device top-k (logits kept, k candidates out)
    for k in (1, 40):
        ti = torch.empty((1, k), dtype=torch.int32, device=dev)
        tv = torch.empty((1, k), device=dev)
        timed(f"c4 q8_0_gemv_topk vocab 128256x3072 b1 k={k}",
              [lambda w=w: qd.q8_0_gemv_topk(w, 3072, 128256, xv, k, logits=ov, top_idx=ti, top_val=tv)
               for w in wvoc],
              q8_bytes(128256, 3072) + 3072 * 4 + 128256 * 4, iters=40)
    # launch cost of an empty kernel (the analogue of an empty submit round trip)
    timed("empty kernel", [lambda: qd.empty_kernel()], 0)


def time_graph(launch, n, stream_holder, torch, warm=3):
    """Mean duration of one launch: `n` calls of launch(i) captured into one
    HIP graph on a dedicated stream (warmed up there first, so per-stream
    library state such as a workspace exists before the capture), replayed
    once untimed and once between HIP events recorded on the replay stream
    (so only device time is measured)."""
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    stream_holder[0] = cs
    with torch.cuda.stream(cs):
        for i in range(warm):
            launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for i in range(n):
            launch(i)
    rs = torch.cuda.current_stream()
    stream_holder[0] = rs
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(rs)
    g.replay()
    e1.record(rs)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / n


def vendor_gemm(args):
    """Reference point for the batched GEMM: the vendor bf16 GEMM (torch.matmul
    on bf16 operands, which ROCm routes to hipBLASLt) at the config-3 shapes,
    C = A W^T with bf16 output (half the output bytes of the library's f32).
    Timed eagerly (events around 200 launches rotating over 8 weights; each
    launch takes longer than its host call); not part of the product path."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    for M in (128, 512):
        for N, K in ((8192, 3072), (3072, 8192)):
            a = torch.randn(M, K, device=dev, dtype=torch.bfloat16, generator=g)
            ws = [torch.randn(N, K, device=dev, dtype=torch.bfloat16, generator=g) * 0.02 for _ in range(8)]
            out = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
            for i in range(20):
                torch.matmul(a, ws[i % 8].t(), out=out)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(200):
                torch.matmul(a, ws[i % 8].t(), out=out)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / 200
            print(json.dumps({"vendor_gemm": "torch.matmul bf16 (hipBLASLt)", "M": M, "N": N, "K": K,
                              "mean_us": round(us, 2), "tflops": round(2.0 * M * N * K / us / 1e6, 1),
                              "pct_bf16_peak": round(100 * 2.0 * M * N * K / us / 1e6 / BF16_PEAK_TFLOPS, 2)}),
                  flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--suite", action="store_true",
                    help="time every workload configuration (one JSON line each) instead of the step")
    ap.add_argument("--only", default="",
                    help="with --suite: time only the workloads whose name starts with this prefix (e.g. 'c3')")
    ap.add_argument("--ceiling", action="store_true",
                    help="time the plain streaming-read kernel at the decode products' byte counts")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the vendor bf16 GEMM (torch.matmul, hipBLASLt) at the batched-GEMM shapes, "
                         "as a reference point")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a 64 MiB device copy (untimed), the known-size reference that "
                         "scales the profiler's HBM byte counters (with the step or with --suite)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is a "
              "single-GPU weight-streaming kernel and no multi-GPU build exists", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    if args.suite:
        suite(args)
        return
    if args.ceiling:
        ceiling(args)
        return
    if args.vendor_gemm:
        vendor_gemm(args)
        return

    import torch

    import quantized_decode_ggml_amd as qd
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    w_host, x_host = make_inputs()
    print(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    print("[bench] fnv1a64 " + json.dumps(fingerprints(w_host, x_host)), file=sys.stderr, flush=True)

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
    sh = [torch.cuda.current_stream()]
    torch.cuda.synchronize()
    if args.calibrate:
        calibration_copy(qd, torch, dev)

    names = ("qkv", "up", "down_residual")

    def single(name, i):
        L = layers[i % LAYERS]
        stream = sh[0]
        if name == "qkv":
            qd.q8_0_qkv(L["wq"], L["wk"], L["wv"], N_IN, N_Q, N_KV, xs["x_qkv"], q_out, k_out, v_out, stream=stream)
        elif name == "up":
            qd.q8_0_gemv(L["up"], N_IN, N_FF, xs["x_up"], out=up_out, stream=stream)
        else:
            qd.q8_0_gemv_residual(L["down"], N_FF, N_IN, xs["x_down"], xs["r_down"], out=down_out, stream=stream)

    def step(i):
        for name in names:
            single(name, i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Exactly args.steps steps (layers rotating) captured into one HIP graph;
    # one untimed replay, then the timed replay.  The Python/ctypes cost of
    # the calls stays out of the timed region.
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    sh[0] = cs
    g_steps = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_steps, stream=cs):
        for i in range(args.steps):
            step(i)
    sh[0] = torch.cuda.current_stream()
    g_steps.replay()
    torch.cuda.synchronize()

    # timed region: args.steps steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same replay between HIP events (device time of the steps alone)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(sh[0])
    g_steps.replay()
    e1.record(sh[0])
    torch.cuda.synchronize()
    device_ms = e0.elapsed_time(e1)
    del g_steps

    # eager steps (one host call per product), for reference
    launches0 = qd.launch_count()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    assert qd.launch_count() - launches0 == 3 * args.steps, "not every product ran in libqdec"

    # each product alone: `steps` launches over the rotated layers in one
    # graph, mean launch duration (launch gaps included, so slightly above
    # the profiler's kernel duration)
    per_kernel = {}
    sb = step_bytes()
    for n in names:
        us = time_graph(lambda i, n=n: single(n, i), args.steps, sh, torch)
        per_kernel[n] = {"mean_us": round(us, 3), "bytes": sb[n], "gbs": round(sb[n] / (us * 1e-6) / 1e9, 1)}
    dom = max(names, key=lambda n: per_kernel[n]["mean_us"])
    achieved = per_kernel[dom]["gbs"]
    traffic, traffic_detail = measured_traffic(dom)

    # batched prefill GEMM on the layers' FFN weights (config-3 shapes)
    gemm = {}
    for B in (128, 512):
        for nm, key, n_out, n_in in (("up 8192x3072", "up", N_FF, N_IN), ("down 3072x8192", "down", N_IN, N_FF)):
            x3 = torch.from_numpy(synth.normal_f32(synth.seed(3, 2) + B, (B, n_in))).to(dev)
            o3 = torch.empty((B, n_out), device=dev)
            us = time_graph(lambda i, key=key, n_in=n_in, n_out=n_out, x3=x3, o3=o3: qd.q8_0_gemm_batched(
                layers[i % LAYERS][key], n_in, n_out, x3, out=o3, stream=sh[0]), 64, sh, torch)
            flops = 2.0 * B * n_out * n_in
            byts = q8_bytes(n_out, n_in) + 4 * B * (n_in + n_out)
            tf = flops / (us * 1e-6) / 1e12
            attain = min(BF16_PEAK_TFLOPS, flops / byts * HBM_PEAK_GBS / 1e3)
            gemm[f"q8_0 {nm} B{B}"] = {"mean_us": round(us, 3), "tflops": round(tf, 1),
                                        "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                                        "frac_roofline": round(tf / attain, 4),
                                        "bound": "mfma" if attain >= BF16_PEAK_TFLOPS else "hbm"}
            del x3, o3

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
            "device_ms_per_step": round(device_ms / args.steps, 5),
            "kernels": per_kernel,
            "launch": f"one hip graph of {args.steps} steps (3 kernels each), replayed once",
            "eager_ms_per_step": round(wall_eager / args.steps * 1e3, 5),
        },
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch", "traffic_detail": traffic_detail},
        "batched_gemm": {"unit": "TFLOP/s", "peak_bf16_tflops": BF16_PEAK_TFLOPS,
                         "launch": "64 graph-replayed launches over the rotated layers", "shapes": gemm},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["cpu_baseline_single_thread"] = cpu_baseline(w_host, x_host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
