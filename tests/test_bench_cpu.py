"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte and FLOP counts behind the roofline, the roofline classification, the
kernel the plan picks per workload, and the rule that counter-derived HBM
traffic is reported only for the kernel source it was measured on."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from quantized_mixture_experts_router_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_decode_algorithmic_bytes():
    # int4 codes two to a byte, one fp32 scale per 64 codes of a row; FC1 rows
    # are the interleaved gate/linear pairs (2 * inter), FC2 rows the hidden size
    w = W.WORKLOADS["decode"]
    counts = np.full(w.experts, 4)
    fc1, fc2 = bench.kernel_work(w, counts)
    E, H, I, T, k = 8, 4096, 14336, 16, 2
    fc1_weights = E * (2 * I) * (H // 2 + (H // 64) * 4)
    fc2_weights = E * H * (I // 2 + (I // 64) * 4)
    assert fc1["weight_bytes"] == fc1_weights
    assert fc1["bytes"] == fc1_weights + T * H * 4 + T * k * I * 4 == 530579456
    assert fc2["bytes"] == fc2_weights + T * k * I * 4 + T * k * H * 4
    assert fc1["flops"] == 2.0 * T * k * 2 * I * H


def test_grouped_matmul_bytes_follow_the_element_type():
    import numpy as np
    w32 = W.GMM_WORKLOADS["gmm_decode_fc1"]
    idx = np.arange(w32.M * w32.S).reshape(w32.M, w32.S) % 5  # 5 of the 8 groups used
    b32 = bench.gmm_work(w32, idx)
    for sfx, eb in (("f16", 2), ("bf16", 2), ("f64", 8)):
        w = W.GMM_WORKLOADS[f"gmm_decode_fc1_{sfx}"]
        b = bench.gmm_work(w, idx)
        assert b["bytes"] * 4 == b32["bytes"] * eb and b["flops"] == b32["flops"]
    used = int(np.unique(idx).size)
    assert b32["weight_bytes"] == used * (w32.K * w32.N + w32.N) * 4


def test_unused_experts_are_not_counted():
    w = W.WORKLOADS["decode"]
    counts = np.array([3, 0, 5, 0, 0, 8, 16, 0])
    fc1, _ = bench.kernel_work(w, counts)
    full, _ = bench.kernel_work(w, np.full(8, 4))
    assert fc1["used_experts"] == 4
    assert fc1["weight_bytes"] * 2 == full["weight_bytes"]


def test_share_work_counts_held_slots():
    # an expert share counts only the slots routed to the experts it holds
    w = W.WORKLOADS["large_e_ep8"]
    counts = np.full(w.held, 512)
    fc1, fc2 = bench.kernel_work(w, counts)
    S = 16 * 512
    assert fc1["flops"] == 2.0 * S * 2 * w.inter * w.hidden
    assert fc2["flops"] == 2.0 * S * w.hidden * w.inter


def test_roofline_bound_follows_intensity():
    # decode FC1: about 14 FLOP/B, far below the f16 ridge (2500 TFLOP/s over
    # 8 TB/s = 312.5 FLOP/B)
    w = W.WORKLOADS["decode"]
    fc1, _ = bench.kernel_work(w, np.full(8, 4))
    r = bench.roofline_for(fc1, 0.1)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - fc1["bytes"] / 1e-4 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4
    # prefill FC1: thousands of FLOP/B, matrix-core bound
    w = W.WORKLOADS["prefill"]
    fc1, _ = bench.kernel_work(w, np.full(8, 1024))
    r = bench.roofline_for(fc1, 4.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["achieved"] - fc1["flops"] / 4e-3 / 1e12) < 0.1


def test_kernel_choice_per_workload():
    # read from the library's own launch plan (host code)
    assert bench.gemm_kernel(W.WORKLOADS["tiny"]) == "qmoe_tiled"         # K = 64: no whole 128-byte items
    # K = 1792: no whole 1024-code stage; 8-row tiles stream it in 256-code K ranges
    assert bench.gemm_kernel(W.WORKLOADS["decode_tp8"], "fc2") == "qmoe_stream"
    assert "tile_rows=8 " in bench.plan_of(W.WORKLOADS["decode_tp8"])
    # the register-tiled GEMM: past the streaming range, I not a multiple of 64
    assert bench.gemm_kernel(W.Workload("odd", (300, 192), 4, 96, 2, 4, 32, "swiglu", (0.005, 0.02))) == "qmoe_gemm"
    assert bench.gemm_kernel(W.WORKLOADS["decode"]) == "qmoe_stream"
    assert bench.gemm_kernel(W.WORKLOADS["decode"], "fc2") == "qmoe_stream"
    assert bench.gemm_kernel(W.WORKLOADS["large_e_ep8"]) == "qmoe_tiled"
    plan = bench.plan_of(W.WORKLOADS["decode"])
    assert "tile_rows=8 " in plan and "s1=1:8:1:2:0" in plan and "s2=1:4:1:14:0" in plan
    for name in ("prefill", "fine", "large_e"):
        assert bench.gemm_kernel(W.WORKLOADS[name]) == "qmoe_tiled"
    # segment scales between the tiled GEMMs: one segment per FC1 column tile
    # (128 SwiGLU codes, 256 ReLU codes)
    assert "segments=112 " in bench.plan_of(W.WORKLOADS["prefill"])
    assert "segments=11 " in bench.plan_of(W.WORKLOADS["fine"])
    assert "segments=12 " in bench.plan_of(W.WORKLOADS["large_e"])
    assert "segments=1 " in bench.plan_of(W.WORKLOADS["tiny"])
    # K ranges of the tiled FC2: four at prefill (about 1100 tiles of 128 x
    # 256 for 256 compute units), one where the reduction is too short to
    # split into ranges of 1024 codes or more
    assert "fc2_ranges=4 " in bench.plan_of(W.WORKLOADS["prefill"])
    for name in ("fine", "large_e", "large_e_ep8", "tiny"):
        assert "fc2_ranges=1 " in bench.plan_of(W.WORKLOADS[name]), name
    assert bench.gmm_kernel(W.GMM_WORKLOADS["gmm_decode_fc1"]) == "qmoe_gmm_f32_rows16"
    assert bench.gmm_kernel(W.GMM_WORKLOADS["gmm_fine_fc1"]) == "qmoe_gmm_f32"
    for sfx in ("f16", "bf16"):
        assert bench.gmm_kernel(W.GMM_WORKLOADS[f"gmm_fine_fc1_{sfx}"]) == "qmoe_gmm16_tiled"
    assert bench.gmm_kernel(W.GMM_WORKLOADS["gmm_fine_fc1_f64"]) == "qmoe_gmm_typed"
    assert bench.gmm_kernel(W.GMM_WORKLOADS["gmm_decode_fc1_f16"]) == "qmoe_gmm16_stream"
    assert bench.gmm_kernel(W.GMM_WORKLOADS["gmm_decode_fc1_bf16"]) == "qmoe_gmm16_stream"
    assert bench.gmm_kernel(W.GMM_WORKLOADS["gmm_decode_fc1_f64"]) == "qmoe_gmm64_rows16"


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    plan = "fc1=stream fc2=stream s1=1:4:1:4:0"
    rec = {"decode:fc1": {"kernel": "qmoe_stream", "source_sha": bench._sha(str(src)), "plan": plan, "bytes": 123}}
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    monkeypatch.setitem(bench.KERNEL_SRC, "qmoe_stream", str(src))
    assert bench.traffic_for("decode:fc1", "qmoe_stream", plan) == 123
    assert bench.traffic_for("decode:fc2", "qmoe_stream", plan) is None      # never measured
    assert bench.traffic_for("decode:fc1", "qmoe_tiled", plan) is None       # another kernel
    assert bench.traffic_for("decode:fc1", "qmoe_stream", "fc1=stream s1=1:4:1:8:0") is None  # another plan
    # the workspace layout moves no bytes: a record stays valid across it
    assert bench.traffic_for("decode:fc1", "qmoe_stream", plan + " segflag=512 workspace=4096") == 123
    assert bench.traffic_for("decode:fc1", "qmoe_stream", plan + " segments=3 workspace=4096") is None
    src.write_text("// kernel source, changed\n")
    assert bench.traffic_for("decode:fc1", "qmoe_stream", plan) is None      # source changed since
