"""CPU checks of the benchmark's accounting: the algorithmic bytes and pairs it
divides by, the stored counter lookup, and the one-GPU guard. No GPU needed."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_progressive_window_amd import build, workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_headline_pairs_per_step():
    # every layer counts N * K_prev candidate pairs per window-head (K_prev = N for
    # the dense layer), over 1440 window-heads and 6 blocks
    w = workloads.MAP640
    assert w.n_wh == 6 * (384 // 32) * (640 // 32) == 1440
    per_block = 1440 * 1024 * (1024 + 1024 + 256 + 128 + 64 + 32)
    assert sum(w.pairs(l) for l in range(w.layers)) * w.blocks == per_block * 6 == 22_366_126_080


def test_fused_all_candidates_bytes():
    # the fused second layer reads both layers' Q and K (bf16) and writes I^2, A^2
    w = workloads.MAP640
    per_wh = 4 * 1024 * 32 * 2 + 1024 * 256 * (4 + 4)
    assert bench.kernel_bytes(w, 1, bench.ALL_CAND, True, True, fused=True) == per_wh
    assert per_wh * w.n_wh == 3_397_386_240
    # dense first layer without A^1: Q, K, V read, O (fp32) written
    assert bench.kernel_bytes(w, 0, bench.DENSE, True, True, fused=True) == 3 * 1024 * 32 * 2 + 1024 * 32 * 4


@pytest.mark.parametrize("name", ["map256x256_h6_d32_f32", "map640x384_h6_d32_bf16_6blocks"])
def test_split_layers_add_up(name):
    # a layer run as selection + aggregation moves the layer's bytes plus one
    # re-read of the kept (I, A) rows by the aggregation
    w = workloads.BY_NAME[name]
    for l in range(2, w.layers):
        sel = bench.kernel_bytes(w, l, bench.SELECT, False, True)
        agg = bench.kernel_bytes(w, l, bench.AGGREGATE, False, True)
        assert sel + agg == bench.layer_bytes(w, l, False) + w.N * w.K[l] * 8
        assert bench.kernel_flops(w, l, bench.SELECT, True) + bench.kernel_flops(w, l, bench.AGGREGATE, True) \
            == 2 * w.d * w.N * (w.K[l - 1] + w.K[l])


def test_stored_traffic_follows_the_source_digest(monkeypatch):
    path = os.path.join(ROOT, "profiles", bench.COUNTERS_FILE.format(workload="map640x384_h6_d32_bf16_6blocks_fused12"))
    text = open(path).read()
    blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    entry = next(k for k in blob["kernels"] if k["kernel"] == "all_cand" and k["layer"] == 2)
    # counters agree with the algorithmic bytes within the measured excess
    for k in blob["kernels"]:
        assert 0.99 <= k["traffic_bytes"] / k["alg_bytes"] <= 1.2, k
    monkeypatch.setattr(build, "source_digest", lambda: blob["source_sha256"])
    assert bench.stored_traffic("map640x384_h6_d32_bf16_6blocks_fused12", "all_cand", 2) == entry["traffic_bytes"]
    monkeypatch.setattr(build, "source_digest", lambda: "0" * 64)
    assert bench.stored_traffic("map640x384_h6_d32_bf16_6blocks_fused12", "all_cand", 2) is None
