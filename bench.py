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
COUNTERS_FILE = "hbm_counters_{workload}.md"

# kernel kinds of the library's timing calls (pfa_kernel_kind)
DENSE, ALL_CAND, SPARSE, SELECT, AGGREGATE, IOTA, BWD_ROWS, BWD_SCATTER, IET_RANK, IET_UNION, DENSE_BWD = range(11)


def kernel_bytes(w, l, kind, i_prev_implicit, split, fused=False):
    """Algorithmic HBM bytes of one launch of kernel `kind` in layer l (0-based),
    per window-head: every input read once, every output written once. `split`:
    the layer ran a separate aggregation kernel, so this one does not touch V or O.
    `fused`: layers 1-2 ran fused (no A^1: the dense layer writes O only, the
    second layer reads the first layer's Q and K instead of A^1)."""
    N, d = w.N, w.d
    b_in = 4 if w.dtype == "f32" else 2
    x = N * d * b_in                      # one of Q, K, V
    O = N * d * 4
    if kind == DENSE:
        return 3 * x + O + (0 if fused else N * N * 4)   # A^1 materialised unless fused; I^1 implicit
    if fused and l == 1 and kind == ALL_CAND:
        return 4 * x + N * w.K[1] * 8
    if kind == IOTA:
        return N * N * 4
    K_prev, K_l = w.K[l - 1], w.K[l]
    I_prev = 0 if i_prev_implicit else N * K_prev * 4
    kept = N * K_l * 8                    # I^l and A^l rows
    if kind == AGGREGATE:
        return x + kept + O
    sel = 2 * x + I_prev + N * K_prev * 4 + kept
    if split:
        return sel
    return sel + x + O


def kernel_flops(w, l, kind, split):
    """Algorithmic flops per window-head: 2d per scored pair, 2d per aggregated pair."""
    N, d = w.N, w.d
    if kind == DENSE:
        return 4 * d * N * N
    if kind == IOTA:
        return 0
    K_prev, K_l = w.K[l - 1], w.K[l]
    if kind == AGGREGATE:
        return 2 * d * N * K_l
    if split:
        return 2 * d * N * K_prev
    return 2 * d * N * K_prev + 2 * d * N * K_l


def bwd_kernel_bytes(w, l, part, i_prev_implicit):
    """Algorithmic HBM bytes per window-head of one backward launch of layer l
    (0-based): each kernel's own inputs read once and outputs written once,
    including the per-pair workspace g. part: "V" (G, g), "K" (dQ, dA^{l-1}),
    "KV" (both in one kernel) or "scatter" (dK, dV from A, g, Q, dO)."""
    N, d = w.N, w.d
    x = N * d * (4 if w.dtype == "f32" else 2)
    f = N * d * 4
    K_prev, K_l = w.K[l - 1], w.K[l]
    pairs = N * K_l * 4
    prev = N * K_prev * 4
    ip = 0 if i_prev_implicit else prev
    dA = pairs if l < w.layers - 1 else 0      # the last layer's map has no consumer
    if part == "V":
        return x + 2 * pairs + dA + f + pairs
    if part == "K":
        return 2 * x + 3 * pairs + ip + prev + f + prev
    if part == "KV":
        return 3 * x + 2 * pairs + dA + f + pairs + ip + prev + f + prev
    return x + 3 * pairs + f + 2 * f


def stored_traffic(workload, kernel, layer):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    from sparse_progressive_window_amd import build
    path = os.path.join(ROOT, "profiles", COUNTERS_FILE.format(workload=workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    if blob.get("source_sha256") != build.source_digest():
        return None
    for k in blob.get("kernels", []):
        if k["kernel"] == kernel and k["layer"] == layer:
            return k["traffic_bytes"]
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="map256x256_h6_d32_f32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=384, help="window-heads timed on the CPU oracle")
    ap.add_argument("--fused12", action="store_true",
                    help="run layers 1-2 fused without materialising A^1 (bf16, or fp32 with d = 16)")
    ap.add_argument("--rpb", action="store_true",
                    help="add a seeded relative position bias table per layer to the scores (not with --fused12)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward leg (layers L..2 of the sparse-layer backward, timed separately)")
    ap.add_argument("--no-global", action="store_true",
                    help="skip the global-mode leg (individualized attention + index propagation, 64x64 map)")
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
    fused = args.fused12
    for l in range(L):
        K_l = w.K[l]
        I = None if l == 0 else torch.empty(lead + (N, K_l), dtype=torch.int32, device=dev)
        A = None if (fused and l == 0) else torch.empty(lead + (N, K_l), dtype=torch.float32, device=dev)
        O = torch.empty((w.B, w.heads, w.H, w.W, w.d), dtype=torch.float32, device=dev)
        outs.append((I, A, O))
    implicit = [l == 1 and w.K[0] == N for l in range(L)]
    bias = [None] * L
    if args.rpb:
        if fused:
            print("--rpb does not combine with --fused12", file=sys.stderr)
            sys.exit(2)
        gb = torch.Generator().manual_seed(777)
        bias = [torch.randn((w.heads, (2 * w.win - 1) ** 2), generator=gb).to(dev) for _ in range(L)]

    def step(marks=None):
        for l in range(L):
            Q, K, V = qkv[l]
            if fused and l == 0:
                pfa.first_two_layers(Q, K, V, *qkv[1], w.K[1], win=w.win, shift1=w.shifts[0], shift2=w.shifts[1],
                                     out=(outs[0][2],) + outs[1])
            elif fused and l == 1:
                pass   # done with layer 1
            elif l == 0:
                pfa.dense_layer(Q, K, V, w.K[0], win=w.win, shift=w.shifts[0], out=outs[0], bias=bias[0])
            else:
                I_prev = None if implicit[l] else outs[l - 1][0]
                pfa.sparse_layer(Q, K, V, I_prev, outs[l - 1][1], w.K[l], win=w.win, shift=w.shifts[l],
                                 out=outs[l], bias=bias[l])
            if marks is not None:
                marks.append(pfa.timing_count())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps; every kernel is bracketed by HIP events on its launch
    # stream (the library's timing calls), read back after the final synchronize.
    pfa.timing_enable(args.steps * L * 2 + 64)
    marks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(marks)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    recs, dropped = pfa.timing_read(len(marks) * 4 + 64)
    pfa.timing_enable(0)
    assert dropped == 0 and len(recs) == marks[-1], (dropped, len(recs), marks[-1])

    # per (layer, kernel kind): launch durations
    per = {}
    start = 0
    for i, end in enumerate(marks):
        l = i % L
        for kind, ms in recs[start:end]:
            ll = 1 if (fused and l == 0 and kind != DENSE) else l   # fused call: dense = layer 1, rest = layer 2
            per.setdefault((ll, kind), []).append(ms)
        start = end
    layer_ms = [sum(float(np.mean(v)) for (ll, _), v in per.items() if ll == l) for l in range(L)]

    layers, kernels = [], []
    total_pairs = 0
    for l in range(L):
        pairs = w.pairs(l)
        total_pairs += pairs
        layers.append({"layer": l + 1, "K_prev": N if l == 0 else w.K[l - 1], "K_l": w.K[l],
                       "ms": round(layer_ms[l], 4), "pairs_per_s": pairs / (layer_ms[l] * 1e-3)})
    peak_mfma = FP32_MFMA_PEAK_TFLOPS if w.dtype == "f32" else BF16_MFMA_PEAK_TFLOPS
    for (l, kind), v in sorted(per.items()):
        ms = float(np.mean(v))
        split = (l, AGGREGATE) in per
        by = kernel_bytes(w, l, kind, implicit[l], split, fused) * w.n_wh
        fl = kernel_flops(w, l, kind, split) * w.n_wh
        gbs = by / (ms * 1e-3) / 1e9
        tfs = fl / (ms * 1e-3) / 1e12
        mfma = kind in (DENSE, ALL_CAND)
        # the bound is whichever roofline time is longer for the algorithmic work
        t_hbm = by / (HBM_PEAK_GBS * 1e9)
        t_mfma = fl / (peak_mfma * 1e12) if mfma else 0.0
        bound = "mfma" if t_mfma > t_hbm else "hbm"
        kernels.append({"layer": l + 1, "kernel": pfa.kernel_name(kind), "launches": len(v), "ms": round(ms, 4),
                        "alg_bytes": by, "GB_per_s": round(gbs, 1), "alg_flops": fl, "TFLOP_per_s": round(tfs, 2),
                        "bound": bound,
                        "frac": round(tfs / peak_mfma if bound == "mfma" else gbs / HBM_PEAK_GBS, 4)})

    dom = max(kernels, key=lambda k: k["ms"])
    if dom["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dom["TFLOP_per_s"], "peak": peak_mfma, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": dom["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = dom["frac"]
    roof["traffic"] = stored_traffic(w.name, dom["kernel"], dom["layer"])
    roof.update({"kernel": dom["kernel"], "layer": dom["layer"], "ms_per_launch": dom["ms"],
                 "alg_bytes_per_launch": dom["alg_bytes"], "alg_flops_per_launch": dom["alg_flops"]})

    value = total_pairs / (ms_per_step * 1e-3)
    result = {
        "metric": "PFA candidate-pairs/sec per layer (32\u00d732 win, d=32); % HBM/MFMA roofline",
        "value": value, "unit": "candidate pairs/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "fused_layers_1_2": fused, "relative_position_bias": bool(args.rpb), "B": w.B, "heads": w.heads, "H": w.H, "W": w.W,
                   "d": w.d, "win": w.win,
                   "K": w.K, "shifts": w.shifts, "window_heads": w.n_wh, "pairs_per_step": total_pairs},
        "roofline": roof, "layers": layers, "kernels": kernels,
    }

    if not args.no_backward and not fused:
        try:
            result["backward"] = backward_leg(w, qkv, outs, implicit, args, torch, pfa)
            if not args.no_cpu_baseline:
                result["backward"]["cpu_baseline"] = cpu_baseline_backward(w, host, outs, implicit)
        except Exception as e:   # the forward line stands on its own
            result["backward"] = {"error": repr(e)}
    if not args.no_global:
        try:
            result["global"] = global_leg(args, torch, pfa)
            if not args.no_cpu_baseline:
                result["global"]["cpu_baseline"] = cpu_baseline_global()
        except Exception as e:   # the forward line stands on its own
            result["global"] = {"error": repr(e)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, host, args.cpu_sample)
    print(json.dumps(result), flush=True)


def backward_leg(w, qkv, outs, implicit, args, torch, pfa):
    """Backward of the whole chain just run: the sparse layers L..2 (kept sets
    from its forward outputs), each taking the next one's dA^{l} output and a
    seeded dO, then the dense first layer with the second layer's dA^1; timed
    like the forward step, per kernel with HIP events."""
    dev = qkv[0][0].device
    L, N = w.layers, w.N
    lead = (w.B, w.heads, w.n_windows)
    g = torch.Generator(device="cpu").manual_seed(4242)
    dO = [torch.randn(qkv[l][0].shape, generator=g).to(dev) for l in range(L)]
    grads = [tuple(torch.empty(qkv[l][0].shape, dtype=torch.float32, device=dev) for _ in range(3))
             for l in range(L)]
    dA_prev = [None] + [torch.empty(lead + (N, w.K[l - 1]), dtype=torch.float32, device=dev) for l in range(1, L)]
    ws = torch.empty(max(pfa.backward_workspace_bytes(qkv[l][0], w.K[l], win=w.win) for l in range(1, L)),
                     dtype=torch.uint8, device=dev)
    # the dense layer's log denominators (its forward in the timed step writes A^1, not these)
    dense_bwd = w.K[0] == N and implicit[1]
    lse = torch.empty(lead + (N,), dtype=torch.float32, device=dev)
    if dense_bwd:
        pfa.dense_layer(*qkv[0], win=w.win, shift=w.shifts[0], want_A=False, lse_out=lse)

    def bstep(marks=None):
        for l in range(L - 1, 0, -1):
            Q, K, V = qkv[l]
            I_prev = None if implicit[l] else outs[l - 1][0]
            dA = dA_prev[l + 1] if l + 1 < L else None
            pfa.sparse_layer_backward(Q, K, V, I_prev, outs[l - 1][1], outs[l][0], outs[l][1], dO[l], dA,
                                      win=w.win, shift=w.shifts[l], K_prev=w.K[l - 1],
                                      out=grads[l] + (dA_prev[l],), workspace=ws)
            if marks is not None:
                marks.append(pfa.timing_count())
        if dense_bwd:
            pfa.dense_layer_backward(*qkv[0], lse, dO[0], dA_prev[1], win=w.win, shift=w.shifts[0], out=grads[0],
                                     workspace=ws)
            if marks is not None:
                marks.append(pfa.timing_count())

    for _ in range(args.warmup):
        bstep()
    torch.cuda.synchronize()
    pfa.timing_enable(args.steps * L * 3 + 64)
    marks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        bstep(marks)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    recs, dropped = pfa.timing_read(len(marks) * 4 + 64)
    pfa.timing_enable(0)
    assert dropped == 0 and len(recs) == marks[-1], (dropped, len(recs), marks[-1])
    per = {}
    start = 0
    nlay = L if dense_bwd else L - 1
    for i, end in enumerate(marks):
        l = L - 1 - (i % nlay)
        if l == 0:
            for kind, ms in recs[start:end]:
                per.setdefault((0, "dense"), []).append(ms)
            start = end
            continue
        rows = [ms for kind, ms in recs[start:end] if kind == BWD_ROWS]
        parts = ["V", "K"] if len(rows) == 2 else ["KV"]
        for part, ms in zip(parts, rows):
            per.setdefault((l, part), []).append(ms)
        for kind, ms in recs[start:end]:
            if kind == BWD_SCATTER:
                per.setdefault((l, "scatter"), []).append(ms)
        start = end
    kernels = []
    for (l, part), v in sorted(per.items()):
        ms = float(np.mean(v))
        if part == "dense":
            # Q, K, V, lse, dO, dA^1 read; dQ, dK, dV written; 5 products of 2 N^2 d flops
            x = N * w.d * (4 if w.dtype == "f32" else 2)
            by = (3 * x + N * 4 + N * w.d * 4 + N * N * 4 + 3 * N * w.d * 4) * w.n_wh
            fl = 10 * N * N * w.d * w.n_wh
            tfs = fl / (ms * 1e-3) / 1e12
            gbs = by / (ms * 1e-3) / 1e9
            mfma = fl / (FP32_MFMA_PEAK_TFLOPS * 1e12) > by / (HBM_PEAK_GBS * 1e9)
            kernels.append({"layer": 1, "kernel": "dense_bwd(dq+dkv)", "launches": len(v), "ms": round(ms, 4),
                            "alg_bytes": by, "GB_per_s": round(gbs, 1), "alg_flops": fl,
                            "TFLOP_per_s": round(tfs, 2), "bound": "mfma" if mfma else "hbm",
                            "frac": round(tfs / FP32_MFMA_PEAK_TFLOPS if mfma else gbs / HBM_PEAK_GBS, 4)})
            continue
        by = bwd_kernel_bytes(w, l, part, implicit[l]) * w.n_wh
        gbs = by / (ms * 1e-3) / 1e9
        name = "bwd_dkv_kernel" if part == "scatter" else f"bwd_rows_kernel({part})"
        k = {"layer": l + 1, "kernel": name, "launches": len(v), "ms": round(ms, 4), "alg_bytes": by,
             "GB_per_s": round(gbs, 1), "bound": "hbm", "frac": round(gbs / HBM_PEAK_GBS, 4)}
        if part == "scatter" and w.N % 16 == 0:
            # dV = A^T dO and dK = (A g)^T Q as dense fp32 MFMA products: 4 N^2 d flops per window-head
            fl = 4 * w.N * w.N * w.d * w.n_wh
            tfs = fl / (ms * 1e-3) / 1e12
            k.update({"alg_flops": fl, "TFLOP_per_s": round(tfs, 2)})
            if fl / (FP32_MFMA_PEAK_TFLOPS * 1e12) > by / (HBM_PEAK_GBS * 1e9):
                k.update({"bound": "mfma", "frac": round(tfs / FP32_MFMA_PEAK_TFLOPS, 4)})
        kernels.append(k)
    layer_ms = {l + 1: round(sum(k["ms"] for k in kernels if k["layer"] == l + 1), 4)
                for l in range(0 if dense_bwd else 1, L)}
    kept = sum(w.n_wh * N * w.K[l] for l in range(0 if dense_bwd else 1, L))
    dom = max(kernels, key=lambda k: k["ms"])
    if dom["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dom["TFLOP_per_s"], "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": dom["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof.update({"frac": dom["frac"], "traffic": None, "kernel": dom["kernel"], "layer": dom["layer"],
                 "ms_per_launch": dom["ms"], "alg_bytes_per_launch": dom["alg_bytes"]})
    return {"ms_per_step": round(ms_per_step, 4), "layers": f"{L}..1" if dense_bwd else f"{L}..2", "layer_ms": layer_ms,
            "kept_pairs_per_s": kept / (ms_per_step * 1e-3), "roofline": roof, "kernels": kernels}


def global_leg(args, torch, pfa):
    """Global individualized attention (one index matrix of k candidates per token,
    shared by the heads; softmax over them; O) on the 64x64 global workload,
    followed by the index propagation with each IET block's (k1, k2). Each
    kernel is timed with HIP events over `steps` repetitions; the whole working
    set (~9 MB) fits the 256 MB MALL, so these are latency-bound figures."""
    from sparse_progressive_window_amd import inputs, workloads
    w = workloads.GLOBAL64
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(t.device.view(np.int16)).to(dev).view(torch.bfloat16) for t in inputs.qkv(w, 0, 0))
    N, kk, H = w.N, w.k_global, w.heads
    Iidx = torch.from_numpy(inputs.global_index(w)).to(dev).view(1, 1, N, kk)
    outs = (torch.empty((1, H, N, kk), dtype=torch.int32, device=dev),
            torch.empty((1, H, N, kk), dtype=torch.float32, device=dev),
            torch.empty(q.shape, dtype=torch.float32, device=dev))
    blocks = list(zip((22, 20, 14, 12), (12, 10, 7, 6)))
    iet_out = [(torch.empty((1, N, k1 + k2 * k2), dtype=torch.int32, device=dev),
                torch.empty((1, N), dtype=torch.int32, device=dev)) for k1, k2 in blocks]
    ws = torch.empty(max(int(pfa.load().pfa_iet_propagate_workspace(1, N, k1, k2)) for k1, k2 in blocks),
                     dtype=torch.uint8, device=dev)
    I_map = Iidx.view(1, N, kk)

    def gstep():
        pfa.sparse_layer(q, k, v, Iidx, None, kk, win=0, i_shared=True, out=outs)
        A4 = outs[1].view(1, H, N, kk)
        for (k1, k2), o in zip(blocks, iet_out):
            pfa.iet_propagate(I_map, A4, k1, k2, out=o, workspace=ws)

    for _ in range(args.warmup):
        gstep()
    torch.cuda.synchronize()
    pfa.timing_enable(args.steps * (1 + 2 * len(blocks)) + 16)
    for _ in range(args.steps):
        gstep()
    torch.cuda.synchronize()
    recs, dropped = pfa.timing_read(args.steps * (1 + 2 * len(blocks)) + 16)
    pfa.timing_enable(0)
    assert dropped == 0
    per = {}
    for kind, ms in recs:
        per.setdefault(kind, []).append(ms)
    attn_bytes = H * (3 * N * w.d * 2 + 2 * N * kk * 4 + N * w.d * 4) + N * kk * 4
    rank_bytes = len(blocks) * (N * kk * 4 + H * N * kk * 4) + sum(N * (k1 + k2) * 4 for k1, k2 in blocks)
    union_bytes = sum(N * (k1 + k2) * 4 + N * (k1 + k2 * k2 + 1) * 4 for k1, k2 in blocks)
    kernels = []
    for kind, by, launches_per_step in ((SPARSE, attn_bytes, 1), (IET_RANK, rank_bytes, len(blocks)),
                                        (IET_UNION, union_bytes, len(blocks))):
        v_ = per.get(kind, [])
        if not v_:
            continue
        ms = float(np.mean(v_)) * launches_per_step      # per step (all blocks)
        gbs = by / (ms * 1e-3) / 1e9
        kernels.append({"kernel": pfa.kernel_name(kind), "launches_per_step": launches_per_step,
                        "ms_per_step": round(ms, 4), "alg_bytes": by, "GB_per_s": round(gbs, 1),
                        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
    pairs = H * N * kk
    attn_ms = next(k_["ms_per_step"] for k_ in kernels if k_["kernel"] == pfa.kernel_name(SPARSE))
    return {"workload": w.name, "pairs": pairs, "attention_pairs_per_s": pairs / (attn_ms * 1e-3),
            "iet_blocks_k1_k2": blocks, "kernels": kernels,
            "note": "working set fits the MALL: latency-bound, HBM fraction not meaningful"}


def cpu_baseline_backward(w, host, outs, implicit, sample=384):
    """fp64 backward oracle on `sample` window-heads of each sparse layer, with
    the GPU forward's kept sets (the backward holds them fixed): kept pairs/s."""
    import oracle
    sel = np.linspace(0, w.n_wh - 1, sample).astype(np.int64)
    N = w.N
    g = np.random.Generator(np.random.PCG64(4243))
    t_total, kept = 0.0, 0
    for l in range(1, w.layers):
        Q, K, V = (t.exact for t in host[l])
        keep = outs[l][0].view(-1, N, w.K[l])[sel].cpu().numpy()
        Ip = None if implicit[l] else outs[l - 1][0].view(-1, N, w.K[l - 1])[sel].cpu().numpy()
        Ap = outs[l - 1][1].view(-1, N, w.K[l - 1])[sel].cpu().numpy()
        dO = g.standard_normal(Q.shape)
        dA = g.standard_normal(keep.shape) if l < w.layers - 1 else None
        t0 = time.perf_counter()
        oracle.layer_backward(Q, K, V, win=w.win, shift=w.shifts[l], keep=keep, dO=dO, dA=dA, I_prev=Ip, A_prev=Ap,
                              prev_compact=True, wh_list=sel)
        t_total += time.perf_counter() - t0
        kept += len(sel) * N * w.K[l]
    return {"value": kept / t_total, "unit": "kept pairs/s (backward, layers 6..2)", "cores": oracle.threads(),
            "kind": "oracle", "sample": f"{len(sel)} of {w.n_wh} window-heads per layer ({kept} kept pairs, "
                                        f"{t_total:.1f} s of oracle time)"}


def cpu_baseline_global():
    """fp64 oracle of the global individualized attention (6 heads) and the
    index propagation of the first IET block, on the whole 64x64 workload."""
    import oracle
    from sparse_progressive_window_amd import inputs, workloads
    w = workloads.GLOBAL64
    Qt, Kt, Vt = inputs.qkv(w, 0, 0)
    Iidx = inputs.global_index(w)
    N, k = w.N, w.k_global
    t_attn, reps = 0.0, 0
    while reps == 0 or (t_attn < 2.0 and reps < 200):   # repeated: one pass takes tens of ms
        t0 = time.perf_counter()
        r = oracle.layer(Qt.exact, Kt.exact, Vt.exact, win=0, shift=0, K_l=k, I_prev=Iidx.reshape(1, 1, 1, N, k),
                         i_shared=True, wh_list=np.arange(w.heads))
        t_attn += time.perf_counter() - t0
        reps += 1
    A = r["A"].astype(np.float32).reshape(w.heads, N, k)
    t0 = time.perf_counter()
    oracle.iet_propagate(Iidx, A, 22, 12)
    t_prop = time.perf_counter() - t0
    return {"value": reps * w.heads * N * k / t_attn, "unit": "candidate pairs/s (global attention)",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"whole workload: attention {reps} times, {t_attn:.2f} s; one propagation (k1 = 22, k2 = 12, "
                      f"single-threaded Python oracle) {t_prop:.2f} s"}


def cpu_baseline(w, host, sample, min_seconds=10.0, max_passes=6):
    """fp64 oracle on `sample` window-heads through the whole chain (same inputs),
    repeated until at least `min_seconds` of oracle time (at most `max_passes`)."""
    import oracle
    sel = np.linspace(0, w.n_wh - 1, min(sample, w.n_wh)).astype(np.int64)
    q64 = [tuple(t.exact.astype(np.float64) for t in layer) for layer in host]
    t_total = 0.0
    pairs = 0
    passes = 0
    while passes < max_passes and (passes == 0 or t_total < min_seconds):
        I_prev = A_prev = None
        for l in range(w.layers):
            Q, K, V = q64[l]
            t0 = time.perf_counter()
            r = oracle.layer(Q, K, V, win=w.win, shift=w.shifts[l], K_l=w.K[l], I_prev=I_prev, A_prev=A_prev,
                             prev_compact=True, wh_list=sel)
            t_total += time.perf_counter() - t0
            pairs += len(sel) * w.N * (w.N if l == 0 else w.K[l - 1])
            I_prev, A_prev = r["I"], r["A"]
            del r
        passes += 1
    return {"value": pairs / t_total, "unit": "candidate pairs/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{len(sel)} of {w.n_wh} window-heads through all {w.layers} layers, {passes} pass{'es' if passes > 1 else ''} "
                      f"({pairs} pairs, {t_total:.1f} s of oracle time)"}


if __name__ == "__main__":
    main()
