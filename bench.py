#!/usr/bin/env python3
"""Benchmark of the PFA layer chain on one MI355X.

One step = one pass of the whole chain (dense layer 1 + sparse layers 2..6)
over the 256x256-map workload (64 windows of 32x32, 6 heads, d = 32, fp32
inputs, keep schedule [1024, 256, 128, 64, 32, 16], shift 16 on every second
layer), inputs resident in HBM, outputs preallocated. Prints one JSON line.

Metric: candidate pairs per second (pairs (i, j in I^{l-1}(i)) evaluated, summed
over the chain's layers, divided by the step time); per-layer figures and the
roofline of the dominant kernel are attached. The CPU baseline times the fp64
oracle on a bounded sample of window-heads of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
BF16_MFMA_PEAK_TFLOPS = 2500.0


def layer_bytes(w, l):
    """Algorithmic HBM bytes of layer l (0-based) per window-head."""
    N, d = w.N, w.d
    b_in = 4 if w.dtype == "f32" else 2
    qkv = 3 * N * d * b_in
    O = N * d * 4
    if l == 0:
        return qkv + O + N * N * 4                   # A^1 materialised (I^1 implicit)
    K_prev, K_l = w.K[l - 1], w.K[l]
    I_prev = 0 if (l == 1 and K_prev == N) else N * K_prev * 4
    return qkv + O + I_prev + N * K_prev * 4 + N * K_l * 8


def layer_flops(w, l):
    """Algorithmic flops per window-head: 2d per candidate pair (score) + 2d per kept pair (A.V)."""
    N, d = w.N, w.d
    K_prev = N if l == 0 else w.K[l - 1]
    return 2 * d * N * K_prev + 2 * d * N * w.K[l]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="map256x256_h6_d32_f32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=64, help="window-heads timed on the CPU oracle")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_progressive_window_amd import inputs, pfa, workloads

    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel() * 4, "copies": 3}), flush=True)
        return

    w = workloads.BY_NAME[args.workload]
    assert w.win, "the chain benchmark needs a window workload"
    pfa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(t):
        if t.dtype == "f32":
            return torch.from_numpy(t.device).to(dev)
        return torch.from_numpy(t.device.view(np.int16)).to(dev).view(torch.bfloat16)

    L = w.layers
    host = [inputs.qkv(w, 0, l) for l in range(L)]
    qkv = [tuple(to_dev(t) for t in layer) for layer in host]
    lead = (w.B, w.heads, w.n_windows)
    N = w.N
    outs = []
    for l in range(L):
        K_l = w.K[l]
        I = None if l == 0 else torch.empty(lead + (N, K_l), dtype=torch.int32, device=dev)
        A = torch.empty(lead + (N, K_l), dtype=torch.float32, device=dev)
        O = torch.empty((w.B, w.heads, w.H, w.W, w.d), dtype=torch.float32, device=dev)
        outs.append((I, A, O))
    stream = torch.cuda.current_stream()

    def step(events=None):
        for l in range(L):
            Q, K, V = qkv[l]
            if events is not None:
                events[l][0].record(stream)
            if l == 0:
                pfa.dense_layer(Q, K, V, w.K[0], win=w.win, shift=w.shifts[0], out=outs[0])
            else:
                I_prev = None if (l == 1 and w.K[0] == N) else outs[l - 1][0]
                pfa.sparse_layer(Q, K, V, I_prev, outs[l - 1][1], w.K[l], win=w.win, shift=w.shifts[l],
                                 out=outs[l])
            if events is not None:
                events[l][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step timing (no per-layer events inside)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-layer timing with HIP events on the launch stream
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)] for _ in range(args.steps)]
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    layer_ms = [float(np.mean([ev[s][l][0].elapsed_time(ev[s][l][1]) for s in range(args.steps)]))
                for l in range(L)]

    layers = []
    total_pairs = 0
    for l in range(L):
        pairs = w.pairs(l)
        total_pairs += pairs
        by = layer_bytes(w, l) * w.n_wh
        fl = layer_flops(w, l) * w.n_wh
        gbs = by / (layer_ms[l] * 1e-3) / 1e9
        layers.append({"layer": l + 1, "K_prev": N if l == 0 else w.K[l - 1], "K_l": w.K[l],
                       "ms": round(layer_ms[l], 4), "pairs_per_s": pairs / (layer_ms[l] * 1e-3),
                       "alg_bytes": by, "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                       "alg_flops": fl, "TFLOP_per_s": round(fl / (layer_ms[l] * 1e-3) / 1e12, 2)})

    dom = max(range(L), key=lambda l: layer_ms[l])
    if dom == 0 and w.dtype == "f32":
        ach = layers[0]["TFLOP_per_s"]
        roof = {"bound": "mfma", "kernel": "dense_layer_kernel<float,32>", "layer": 1, "achieved": ach,
                "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / FP32_MFMA_PEAK_TFLOPS, 4),
                "traffic": None}
    else:
        ach = layers[dom]["GB_per_s"]
        roof = {"bound": "hbm", "kernel": "dense_layer_kernel" if dom == 0 else "sparse_layer_kernel",
                "layer": dom + 1, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}

    value = total_pairs / (ms_per_step * 1e-3)
    result = {
        "metric": "PFA candidate-pairs/sec per layer (32x32 win, d=32); % HBM/MFMA roofline",
        "value": value, "unit": "candidate pairs/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "heads": w.heads, "H": w.H, "W": w.W, "d": w.d, "win": w.win,
                   "K": w.K, "shifts": w.shifts, "window_heads": w.n_wh, "pairs_per_step": total_pairs},
        "layers": layers, "roofline": roof,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, host, args.cpu_sample)
    print(json.dumps(result), flush=True)


def cpu_baseline(w, host, sample):
    """fp64 oracle on `sample` window-heads through the whole chain (same inputs)."""
    import oracle
    sel = np.linspace(0, w.n_wh - 1, sample).astype(np.int64)
    q64 = [tuple(t.exact.astype(np.float64) for t in layer) for layer in host]
    I_prev = A_prev = None
    t_total = 0.0
    pairs = 0
    for l in range(w.layers):
        Q, K, V = q64[l]
        t0 = time.perf_counter()
        r = oracle.layer(Q, K, V, win=w.win, shift=w.shifts[l], K_l=w.K[l], I_prev=I_prev, A_prev=A_prev,
                         prev_compact=True, wh_list=sel)
        t_total += time.perf_counter() - t0
        pairs += len(sel) * w.N * (w.N if l == 0 else w.K[l - 1])
        I_prev, A_prev = r["I"], r["A"]
    return {"value": pairs / t_total, "unit": "candidate pairs/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{len(sel)} of {w.n_wh} window-heads through all {w.layers} layers "
                      f"({pairs} pairs, {t_total:.1f} s of oracle time)"}


if __name__ == "__main__":
    main()
