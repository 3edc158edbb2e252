#!/usr/bin/env python3
"""Benchmark of the PFA layer chain on one MI355X.

Headline: the 640x384 inference map (240 windows of 32x32, 6 heads, d = 32,
bf16 inputs), a chain of 6 blocks of 6 layers each (keep schedule [1024, 256,
128, 64, 32, 16] per block, shift 16 on every second layer, fresh Q/K/V per
layer and block). One step = all 36 layer calls; inputs resident in HBM, outputs
preallocated. The first two layers of each block run fused (layer 1 writes O,
layer 2 ranks by exp(s1 + s2); the first layer's map is never materialised),
which is the library's path for bf16 chains; `--unfused` writes A^1 instead.
Prints one JSON line.

Metric: candidate pairs per second (pairs (i, j in I^{l-1}(i)) evaluated, summed
over every layer of the step, divided by the step time). Attached: per-layer
times against the layer's algorithmic bytes (inputs read once, outputs written
once) or flops, per-kernel figures, the roofline of the longest kernel, the
same chain unfused, the 256x256 fp32 map and the 32-image bf16 patch batch as
extra workloads, the backward pass, the global individualized attention, and
the fp64 CPU oracle timed on a bounded sample of the headline workload.
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
HEADLINE = "map640x384_h6_d32_bf16_6blocks"

# kernel kinds of the library's timing calls (pfa_kernel_kind)
(DENSE, ALL_CAND, SPARSE, SELECT, AGGREGATE, IOTA, BWD_ROWS, BWD_SCATTER, IET_RANK, IET_UNION, DENSE_BWD,
 BWD_EXACT, DBIAS, FIRST_MAP) = range(14)
FUSED_BWD_KINDS = {FIRST_MAP: "first_map_and_spread", BWD_ROWS: "bwd_rows", BWD_EXACT: "bwd_exact", BWD_SCATTER: "bwd_dkv",
                   DENSE_BWD: "dense_bwd"}


def kernel_bytes(w, l, kind, i_prev_implicit, split, fused=False):
    """HBM bytes of one launch of kernel `kind` in layer l (0-based) per
    window-head: the kernel's own inputs read once and outputs written once.
    `split`: the layer ran a separate aggregation kernel, so this one does not
    touch V or O (the aggregation kernel's own inputs then include the I^l/A^l
    rows the selection kernel wrote). `fused`: layers 1-2 ran fused (no A^1: the
    dense layer writes O only, the second layer reads the first layer's Q and K
    instead of A^1)."""
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


def kernel_flops(w, l, kind, split, fused=False):
    """Algorithmic flops per window-head: 2d per scored pair (two products of d
    for the fused second layer, q1.k1 + q2.k2), 2d per aggregated pair."""
    N, d = w.N, w.d
    if kind == DENSE:
        return 4 * d * N * N
    if kind == IOTA:
        return 0
    K_prev, K_l = w.K[l - 1], w.K[l]
    if kind == AGGREGATE:
        return 2 * d * N * K_l
    score = (4 if (fused and l == 1 and kind == ALL_CAND) else 2) * d * N * K_prev
    if split:
        return score
    return score + 2 * d * N * K_l


def layer_bytes(w, l, i_prev_implicit, fused=False):
    """Algorithmic bytes of layer l (0-based) per window-head, whatever kernels
    run it: Q, K, V and the previous map read once, I^l, A^l and O written once.
    Dense layer: A^1 written unless fused (then O only). Fused second layer: the
    first layer's Q and K replace the A^1 read."""
    N, d = w.N, w.d
    x = N * d * (4 if w.dtype == "f32" else 2)
    O = N * d * 4
    if l == 0:
        return 3 * x + O + (0 if fused else N * N * 4)
    K_prev, K_l = w.K[l - 1], w.K[l]
    prev = 2 * x if (fused and l == 1) else (0 if i_prev_implicit else N * K_prev * 4) + N * K_prev * 4
    return 3 * x + prev + N * K_l * 8 + O


def mfma_peak(w):
    return FP32_MFMA_PEAK_TFLOPS if w.dtype == "f32" else BF16_MFMA_PEAK_TFLOPS


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
    flags = N * 4                             # one row flag for the exact dA^{l-1} pass
    if part == "K":
        return 2 * x + 3 * pairs + ip + prev + f + prev + flags
    if part == "KV":
        return 3 * x + 2 * pairs + dA + f + pairs + ip + prev + f + prev + flags
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Chain:
    """Device inputs and outputs of one chain workload: Q/K/V per (block, layer),
    output buffers per layer shared by the blocks (each block's chain is
    independent of the others and overwrites them)."""

    def __init__(self, w, torch, pfa, inputs, dev, fused, rpb=False, keep_host_block=None, share=None):
        self.w, self.torch, self.pfa, self.fused = w, torch, pfa, fused
        L, N = w.layers, w.N
        self.host = None

        def to_dev(t):
            if t.dtype == "f32":
                return torch.from_numpy(t.device).to(dev)
            return torch.from_numpy(t.device.view(np.int16)).to(dev).view(torch.bfloat16)

        self.qkv = [] if share is None else share.qkv   # share: another chain's inputs of the same workload
        for b in range(w.blocks if share is None else 0):
            layers = []
            hl = []
            for l in range(L):
                ts = inputs.qkv(w, b, l)
                layers.append(tuple(to_dev(t) for t in ts))
                if keep_host_block == b:
                    hl.append(ts)
            self.qkv.append(layers)
            if keep_host_block == b:
                self.host = hl
        lead = (w.B, w.heads, w.n_windows)
        self.outs = []
        for l in range(L):
            K_l = w.K[l]
            I = None if l == 0 else torch.empty(lead + (N, K_l), dtype=torch.int32, device=dev)
            A = None if (fused and l == 0) else torch.empty(lead + (N, K_l), dtype=torch.float32, device=dev)
            O = torch.empty((w.B, w.heads, w.H, w.W, w.d), dtype=torch.float32, device=dev)
            self.outs.append((I, A, O))
        self.implicit = [l == 1 and w.K[0] == N for l in range(L)]
        self.bias = [None] * L
        if rpb:
            gb = torch.Generator().manual_seed(777)
            self.bias = [torch.randn((w.heads, (2 * w.win - 1) ** 2), generator=gb).to(dev) for _ in range(L)]

    def block(self, b, marks=None):
        w, pfa, outs = self.w, self.pfa, self.outs
        for l in range(w.layers):
            Q, K, V = self.qkv[b][l]
            if self.fused and l == 0:
                pfa.first_two_layers(Q, K, V, *self.qkv[b][1], w.K[1], win=w.win, shift1=w.shifts[0],
                                     shift2=w.shifts[1], out=(outs[0][2],) + outs[1])
            elif self.fused and l == 1:
                pass   # done with layer 1
            elif l == 0:
                pfa.dense_layer(Q, K, V, w.K[0], win=w.win, shift=w.shifts[0], out=outs[0], bias=self.bias[0])
            else:
                I_prev = None if self.implicit[l] else outs[l - 1][0]
                pfa.sparse_layer(Q, K, V, I_prev, outs[l - 1][1], w.K[l], win=w.win, shift=w.shifts[l],
                                 out=outs[l], bias=self.bias[l])
            if marks is not None:
                marks.append(pfa.timing_count())

    def step(self, marks=None):
        for b in range(self.w.blocks):
            self.block(b, marks)


def run_chain(chain, steps, warmup, torch, pfa):
    """Time `steps` chain steps after `warmup`; per-kernel durations from the
    library's HIP events. Returns the result dict (no CPU baseline)."""
    w, fused = chain.w, chain.fused
    L, N = w.layers, w.N
    for _ in range(warmup):
        chain.step()
    torch.cuda.synchronize()

    # Timed region: K steps; every kernel is bracketed by HIP events on its launch
    # stream (the library's timing calls), read back after the final synchronize.
    pfa.timing_enable(steps * w.blocks * L * 2 + 64)
    marks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        chain.step(marks)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
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

    peak_mfma = mfma_peak(w)
    layers, kernels = [], []
    total_pairs = 0
    for l in range(L):
        pairs = w.pairs(l) * w.blocks
        total_pairs += pairs
        by = layer_bytes(w, l, chain.implicit[l], fused) * w.n_wh
        gbs = by / (layer_ms[l] * 1e-3) / 1e9
        ent = {"layer": l + 1, "K_prev": N if l == 0 else w.K[l - 1], "K_l": w.K[l],
               "ms_per_block": round(layer_ms[l], 4), "pairs_per_s": w.pairs(l) / (layer_ms[l] * 1e-3),
               "alg_bytes_per_block": by, "GB_per_s": round(gbs, 1)}
        if l == 0 and fused:
            # O-only dense layer: 4 N^2 d flops per window-head against the MFMA peak
            fl = 4 * w.d * N * N * w.n_wh
            tfs = fl / (layer_ms[l] * 1e-3) / 1e12
            ent.update({"bound": "mfma", "alg_flops_per_block": fl, "TFLOP_per_s": round(tfs, 2),
                        "frac": round(tfs / peak_mfma, 4), "peak": peak_mfma})
        else:
            ent.update({"bound": "hbm", "frac": round(gbs / HBM_PEAK_GBS, 4), "peak": HBM_PEAK_GBS})
        layers.append(ent)
    for (l, kind), v in sorted(per.items()):
        ms = float(np.mean(v))
        split = (l, AGGREGATE) in per
        by = kernel_bytes(w, l, kind, chain.implicit[l], split, fused) * w.n_wh
        fl = kernel_flops(w, l, kind, split, fused) * w.n_wh
        gbs = by / (ms * 1e-3) / 1e9
        tfs = fl / (ms * 1e-3) / 1e12
        mfma = kind in (DENSE, ALL_CAND)
        # the bound is whichever roofline time is longer for the algorithmic work
        t_hbm = by / (HBM_PEAK_GBS * 1e9)
        t_mfma = fl / (peak_mfma * 1e12) if mfma else 0.0
        bound = "mfma" if t_mfma > t_hbm else "hbm"
        k = {"layer": l + 1, "kernel": pfa.kernel_name(kind), "launches": len(v), "ms": round(ms, 4),
             "io_bytes": by, "GB_per_s": round(gbs, 1), "alg_flops": fl, "TFLOP_per_s": round(tfs, 2),
             "bound": bound, "frac": round(tfs / peak_mfma if bound == "mfma" else gbs / HBM_PEAK_GBS, 4)}
        if kind == DENSE and w.dtype == "f32":
            # fp32 inputs run the scores as a three-way bf16 split on bf16 MFMA: also
            # state the fraction of the bf16 peak, the dense-layer target's unit
            k["frac_of_bf16_mfma_peak"] = round(tfs / BF16_MFMA_PEAK_TFLOPS, 4)
        kernels.append(k)

    dom = max(kernels, key=lambda k: k["ms"])
    if dom["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dom["TFLOP_per_s"], "peak": peak_mfma, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": dom["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = dom["frac"]
    roof["traffic"] = stored_traffic(w.name + ("_fused12" if fused else ""), dom["kernel"], dom["layer"])
    roof.update({"kernel": dom["kernel"], "layer": dom["layer"], "ms_per_launch": dom["ms"],
                 "alg_bytes_per_launch": dom["io_bytes"], "alg_flops_per_launch": dom["alg_flops"]})
    chain_bytes = sum(x["alg_bytes_per_block"] for x in layers) * w.blocks
    return {
        "value": total_pairs / (ms_per_step * 1e-3), "ms_per_step": round(ms_per_step, 4),
        "config": {"workload": w.name, "fused_layers_1_2": fused,
                   "relative_position_bias": chain.bias[0] is not None, "B": w.B, "heads": w.heads, "H": w.H,
                   "W": w.W, "d": w.d, "win": w.win, "blocks": w.blocks, "K": w.K, "shifts": w.shifts,
                   "window_heads_per_layer": w.n_wh, "pairs_per_step": total_pairs},
        "chain_alg_bytes_per_step": chain_bytes,
        "chain_GB_per_s": round(chain_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": roof, "layers": layers, "kernels": kernels,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--unfused", action="store_true",
                    help="headline chain with A^1 written and read back (the fused first two layers need bf16, "
                         "or fp32 with d = 16)")
    ap.add_argument("--rpb", action="store_true",
                    help="add a seeded relative position bias table per layer to the scores (unfused only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=384, help="window-heads timed on the CPU oracle")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra workloads (unfused headline, 256x256 fp32 map, bf16 patch batch)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward leg (layers L..1 of the chain's backward, timed separately)")
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
    fusable = w.N == 1024 and (w.dtype == "bf16" or w.d == 16)
    fused = fusable and not args.unfused and not args.rpb

    log(f"generating {w.name} ({w.blocks} blocks x {w.layers} layers)")
    chain = Chain(w, torch, pfa, inputs, dev, fused, rpb=args.rpb, keep_host_block=0)
    log(f"timing {w.name} fused={fused}: {args.warmup} warmup + {args.steps} steps")
    res = run_chain(chain, args.steps, args.warmup, torch, pfa)
    result = {
        "metric": "PFA candidate-pairs/sec per layer (32×32 win, d=32); % HBM/MFMA roofline",
        "value": res.pop("value"), "unit": "candidate pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
    }
    result.update(res)
    log(f"{w.name}: {result['ms_per_step']} ms/step, {result['value']:.3e} pairs/s")

    extras = {}
    if not args.no_extras:
        if fused:
            log(f"timing {w.name} unfused")
            cu = Chain(w, torch, pfa, inputs, dev, False, share=chain)
            extras["unfused"] = run_chain(cu, args.steps, args.warmup, torch, pfa)
            log(f"unfused: {extras['unfused']['ms_per_step']} ms/step")
            if not args.no_backward:
                try:
                    extras["unfused"]["backward"] = backward_leg(cu, args, torch, pfa)
                except Exception as e:   # the forward line stands on its own
                    extras["unfused"]["backward"] = {"error": repr(e)}
            del cu
            torch.cuda.empty_cache()
        for name in ("map256x256_h6_d32_f32", "patch64x64_b32_h6_d32_bf16"):
            if name == w.name:
                continue
            wx = workloads.BY_NAME[name]
            fx = wx.N == 1024 and (wx.dtype == "bf16" or wx.d == 16)
            log(f"timing {name} fused={fx}")
            cx = Chain(wx, torch, pfa, inputs, dev, fx)
            extras[name] = run_chain(cx, args.steps, args.warmup, torch, pfa)
            if not fx and not args.no_backward:
                try:
                    extras[name]["backward"] = backward_leg(cx, args, torch, pfa)
                except Exception as e:
                    extras[name]["backward"] = {"error": repr(e)}
            log(f"{name}: {extras[name]['ms_per_step']} ms/step")
            del cx
            torch.cuda.empty_cache()
    if not args.no_backward:
        try:
            result["backward"] = backward_leg(chain, args, torch, pfa)
        except Exception as e:
            result["backward"] = {"error": repr(e)}
    if extras:
        result["extra_workloads"] = extras
    if not args.no_global:
        try:
            log("timing the global individualized attention")
            result["global"] = global_leg(args, torch, pfa)
            if not args.no_cpu_baseline:
                result["global"]["cpu_baseline"] = cpu_baseline_global()
        except Exception as e:   # the forward line stands on its own
            result["global"] = {"error": repr(e)}
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle")
        result["cpu_baseline"] = cpu_baseline(w, chain.host, args.cpu_sample)
    print(json.dumps(result), flush=True)


def backward_leg(chain, args, torch, pfa):
    """Backward of the last block of the chain just run (its outputs are the ones
    left in the buffers): the sparse layers L..2 (kept sets from the forward
    outputs), each taking the next one's dA^{l} output and a seeded dO, then the
    dense first layer with the second layer's dA^1 (a fused chain: layers L..3,
    then the fused first two layers' backward); timed like the forward step,
    per kernel with HIP events."""
    w, outs, implicit = chain.w, chain.outs, chain.implicit
    qkv = chain.qkv[w.blocks - 1]
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
    fused = chain.fused
    lse = torch.empty(lead + (N,), dtype=torch.float32, device=dev)
    ws_f = None
    if fused:   # the same forward again, now with lse1 (its outputs are bit-identical)
        pfa.first_two_layers(*qkv[0], *qkv[1], w.K[1], win=w.win, shift1=w.shifts[0], shift2=w.shifts[1],
                             out=(outs[0][2],) + outs[1], lse_out=lse)
        ws_f = torch.empty(pfa.first_two_layers_backward_workspace_bytes(qkv[0][0], w.K[1], win=w.win),
                           dtype=torch.uint8, device=dev)
    elif dense_bwd:
        pfa.dense_layer(*qkv[0], win=w.win, shift=w.shifts[0], want_A=False, lse_out=lse)

    def bstep(marks=None):
        for l in range(L - 1, 1 if fused else 0, -1):
            Q, K, V = qkv[l]
            I_prev = None if implicit[l] else outs[l - 1][0]
            dA = dA_prev[l + 1] if l + 1 < L else None
            pfa.sparse_layer_backward(Q, K, V, I_prev, outs[l - 1][1], outs[l][0], outs[l][1], dO[l], dA,
                                      win=w.win, shift=w.shifts[l], K_prev=w.K[l - 1],
                                      out=grads[l] + (dA_prev[l],), workspace=ws)
            if marks is not None:
                marks.append(pfa.timing_count())
        if fused:
            pfa.first_two_layers_backward(*qkv[0], *qkv[1], lse, outs[1][0], outs[1][1], dO[0], dO[1], dA_prev[2],
                                          win=w.win, shift1=w.shifts[0], shift2=w.shifts[1],
                                          out=grads[0] + grads[1], workspace=ws_f)
            if marks is not None:
                marks.append(pfa.timing_count())
        elif dense_bwd:
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
    nlay = L - 1 if fused else L if dense_bwd else L - 1
    for i, end in enumerate(marks):
        l = L - 1 - (i % nlay)
        if fused and l == 1:   # the fused pair: its kernels by kind, summed per call
            acc = {}
            for kind, ms in recs[start:end]:
                key = FUSED_BWD_KINDS.get(kind, str(kind))
                acc[key] = acc.get(key, 0.0) + ms
            for key, ms in acc.items():
                per.setdefault((1, f"fused12:{key}"), []).append(ms)
            start = end
            continue
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
            elif kind == BWD_EXACT:
                per.setdefault((l, "exact"), []).append(ms)
        start = end
    kernels = []
    for (l, part), v in sorted(per.items()):
        ms = float(np.mean(v))
        if part.startswith("fused12:"):
            # per window-head work of the pieces: the first map at the kept pairs (N K2
            # scores), the second layer's row / dK dV passes, the dense layer's backward
            k = {"layer": "1-2", "kernel": part, "launches": len(v), "ms": round(ms, 4)}
            if part.endswith("dense_bwd"):
                x = N * w.d * (4 if w.dtype == "f32" else 2)
                by = (3 * x + N * 4 + N * w.d * 4 + N * N * 4 + 3 * N * w.d * 4) * w.n_wh
                fl = 10 * N * N * w.d * w.n_wh
                k.update({"io_bytes": by, "alg_flops": fl, "TFLOP_per_s": round(fl / (ms * 1e-3) / 1e12, 2),
                          "bound": "mfma", "frac": round(fl / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4)})
            kernels.append(k)
            continue
        if part == "dense":
            # Q, K, V, lse, dO, dA^1 read; dQ, dK, dV written; 5 products of 2 N^2 d flops
            x = N * w.d * (4 if w.dtype == "f32" else 2)
            by = (3 * x + N * 4 + N * w.d * 4 + N * N * 4 + 3 * N * w.d * 4) * w.n_wh
            fl = 10 * N * N * w.d * w.n_wh
            tfs = fl / (ms * 1e-3) / 1e12
            gbs = by / (ms * 1e-3) / 1e9
            mfma = fl / (FP32_MFMA_PEAK_TFLOPS * 1e12) > by / (HBM_PEAK_GBS * 1e9)
            kernels.append({"layer": 1, "kernel": "dense_bwd(dq+dkv)", "launches": len(v), "ms": round(ms, 4),
                            "io_bytes": by, "GB_per_s": round(gbs, 1), "alg_flops": fl,
                            "TFLOP_per_s": round(tfs, 2), "bound": "mfma" if mfma else "hbm",
                            "frac": round(tfs / FP32_MFMA_PEAK_TFLOPS if mfma else gbs / HBM_PEAK_GBS, 4)})
            continue
        if part == "exact":
            # reads one flag per row; rows that need the exact dA^{l-1} pass are rare
            kernels.append({"layer": l + 1, "kernel": "bwd_exact_dap_kernel", "launches": len(v), "ms": round(ms, 4),
                            "io_bytes": N * 4 * w.n_wh, "bound": "latency"})
            continue
        by = bwd_kernel_bytes(w, l, part, implicit[l]) * w.n_wh
        gbs = by / (ms * 1e-3) / 1e9
        name = "bwd_dkv" if part == "scatter" else f"bwd_rows_kernel({part})"
        k = {"layer": l + 1, "kernel": name, "launches": len(v), "ms": round(ms, 4), "io_bytes": by,
             "GB_per_s": round(gbs, 1), "bound": "hbm", "frac": round(gbs / HBM_PEAK_GBS, 4)}
        if part == "scatter":
            # the method's own work: dV = A^T dO and dK = (A g)^T Q over the kept pairs,
            # 4 d flops per kept pair; the bound is whichever roofline time is longer
            fl = 4 * w.d * N * w.K[l] * w.n_wh
            tfs = fl / (ms * 1e-3) / 1e12
            k.update({"alg_flops": fl, "TFLOP_per_s": round(tfs, 2)})
            if fl / (FP32_MFMA_PEAK_TFLOPS * 1e12) > by / (HBM_PEAK_GBS * 1e9):
                k.update({"bound": "mfma", "frac": round(tfs / FP32_MFMA_PEAK_TFLOPS, 4)})
        kernels.append(k)
    if fused:
        layer_ms = {l + 1: round(sum(k["ms"] for k in kernels if k["layer"] == l + 1), 4) for l in range(2, L)}
        layer_ms["1-2"] = round(sum(k["ms"] for k in kernels if k["layer"] == "1-2"), 4)
    else:
        layer_ms = {l + 1: round(sum(k["ms"] for k in kernels if k["layer"] == l + 1), 4)
                    for l in range(0 if dense_bwd else 1, L)}
    kept = sum(w.n_wh * N * w.K[l] for l in range(0 if (dense_bwd or fused) else 1, L))
    dom = max((k for k in kernels if "bound" in k), key=lambda k: k["ms"])
    if dom["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dom["TFLOP_per_s"], "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": dom["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof.update({"frac": dom["frac"], "traffic": None, "kernel": dom["kernel"], "layer": dom["layer"],
                 "ms_per_launch": dom["ms"], "alg_bytes_per_launch": dom["io_bytes"]})
    return {"ms_per_step": round(ms_per_step, 4), "block": w.blocks - 1,
            "layers": f"{L}..3 then fused 2..1" if fused else f"{L}..1" if dense_bwd else f"{L}..2",
            "layer_ms": layer_ms,
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


def host_cpu():
    """Model name, physical cores and the logical CPUs this process may use."""
    model, phys = "unknown", set()
    try:
        cur = {}
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if "core id" in cur:
                        phys.add((cur.get("physical id", "0"), cur["core id"]))
                    cur = {}
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                cur[k] = v
                if k == "model name":
                    model = v
        if "core id" in cur:
            phys.add((cur.get("physical id", "0"), cur["core id"]))
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"model": model, "physical_cores": len(phys) or None, "usable_logical_cpus": usable}


def _oracle_chain_time(w, q64, sel, min_seconds, max_passes, oracle):
    t_total, pairs, passes = 0.0, 0, 0
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
    return t_total, pairs, passes


def cpu_baseline(w, host, sample, min_seconds=10.0, max_passes=6):
    """fp64 oracle on `sample` window-heads of the first block through all its
    layers (same inputs), repeated until at least `min_seconds` of oracle time
    (at most `max_passes`), on every OpenMP thread; then a smaller sample on one
    thread."""
    import oracle
    q64 = [tuple(t.exact.astype(np.float64) for t in layer) for layer in host]
    threads = oracle.threads()
    sel = np.linspace(0, w.n_wh - 1, min(sample, w.n_wh)).astype(np.int64)
    t_total, pairs, passes = _oracle_chain_time(w, q64, sel, min_seconds, max_passes, oracle)
    # one thread: a sample sized for a few seconds at the measured per-thread rate
    per_wh = pairs / passes / len(sel)
    rate1_guess = pairs / t_total / max(threads, 1)
    n1 = int(max(4, min(len(sel), 5.0 * rate1_guess / per_wh)))
    sel1 = np.linspace(0, w.n_wh - 1, n1).astype(np.int64)
    oracle.set_threads(1)
    try:
        t1, pairs1, passes1 = _oracle_chain_time(w, q64, sel1, 3.0, 1, oracle)
    finally:
        oracle.set_threads(threads)
    return {"value": pairs / t_total, "unit": "candidate pairs/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(sel)} of {w.n_wh} window-heads of block 0 through all {w.layers} layers, {passes} "
                      f"pass{'es' if passes > 1 else ''} ({pairs} pairs, {t_total:.1f} s of oracle time)",
            "one_thread": {"value": pairs1 / t1, "cores": 1,
                           "sample": f"{n1} window-heads of block 0, all {w.layers} layers ({pairs1} pairs, "
                                     f"{t1:.1f} s)"},
            "host": host_cpu()}


if __name__ == "__main__":
    main()
