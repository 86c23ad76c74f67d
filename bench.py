#!/usr/bin/env python3
"""QMoE layer benchmark on one AMD Instinct MI355X (gfx950).

One step = one full qmoe_forward (router, permutation, operand prep, FC1 +
activation, FC2, combine) over one batch of seeded synthetic input already
resident in HBM.  Before the W warm-up steps, steps run back to back for
--settle-ms of wall time (untimed) so that the GPU is at its steady clocks;
then exactly K steps are timed.  Default workload: the Mixtral-like int4
decode layer (16 tokens x hidden 4096, 8 experts, inter 14336, k = 2,
interleaved SwiGLU, block size 64); the same JSON line also carries the
prefill layer (2 x 2048 tokens, same experts, block size 128) under
"prefill", timed the same way.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

Workloads named gmm_* measure the standalone float32 GroupedMatMul instead
(one step = one qmoe_grouped_matmul call; roofline of its tile GEMM against
the fp32 matrix peak or HBM), and moe_* the float MoE operator (one step =
one qmoe_moe_forward; roofline of its slower projection).

The roofline object describes the dominant kernel (FC1 or FC2, whichever is
slower), timed with HIP events recorded on the launch stream around that
kernel over K further steps; its algorithmic bytes and FLOPs are counted from
the shapes (packed weights and scales of the experts that receive a slot,
activations in and out).  latency_ms gives per-call median / p10 / p90 with
warm caches and with L2 and the Infinity Cache flushed before every call.
The CPU baseline times the float64 oracle on the host cores over a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
F16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense f16 matrix peak, TFLOP/s
F32_MATRIX_PEAK_TFLOPS = 157.3  # MI355X fp32 matrix (and vector) peak, TFLOP/s
F64_MATRIX_PEAK_TFLOPS = 78.6   # MI355X fp64 matrix peak, TFLOP/s
# GroupedMatMul element types: bytes, matrix peak of the instruction the
# library runs them on, and the short name of the JSON line
GMM_TYPES = {
    "float32": (4, F32_MATRIX_PEAK_TFLOPS, "f32"),
    "float16": (2, F16_DENSE_PEAK_TFLOPS, "f16"),
    "bfloat16": (2, F16_DENSE_PEAK_TFLOPS, "bf16"),  # bf16 dense MFMA: the f16 rate
    "float64": (8, F64_MATRIX_PEAK_TFLOPS, "f64"),
}
METRIC = "QMoE layer tokens/s + achieved HBM GB/s vs peak (int4 decode & prefill)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 warm-up steps bring the GPU to steady clocks (50 steps after 10
    # measured 10-15 % slower per step at the decode workload than longer runs)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="untimed back-to-back steps for this long before the warm-up (steady GPU clocks)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode workload only: skip the prefill entry of the JSON line")
    ap.add_argument("--prefill-steps", type=int, default=0,
                    help="timed steps of the prefill entry (default: the decode steps, clamped to 10..40)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stage-timing", action="store_true")
    ap.add_argument("--no-latency", action="store_true", help="skip the per-call warm/cold latency percentiles")
    ap.add_argument("--crossover", default="", metavar="T1,T2,...",
                    help="time the weight-streaming and the tiled GEMM paths (QMOE_PATH) on the decode layer's "
                         "experts at these token counts; one JSON line")
    ap.add_argument("--layer", default="decode", choices=["decode", "fine", "large_e", "decode_tp8"],
                    help="with --crossover: whose experts and routing recipe (the first T tokens of it)")
    ap.add_argument("--tile-rows", action="store_true",
                    help="with --crossover: also the streaming path with 32-, 48- and 64-row tiles")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    return ap.parse_args()


def kernel_work(w, counts):
    """Algorithmic bytes and FLOPs of the FC1 and FC2 kernels for one call."""
    import numpy as np
    used = int(np.count_nonzero(counts))
    T, H, E, I, k = w.tokens, w.hidden, w.experts, w.inter, w.k
    S = int(np.sum(counts))  # slots on the experts the weights hold (all T * k slots unless a share)
    F = w.fusion * I
    nb1 = H // w.block_size if w.block_size else 1
    nb2 = I // w.block_size if w.block_size else 1
    w1 = used * (F * H // w.pack + F * nb1 * 4)
    w2 = used * (H * I // w.pack + H * nb2 * 4)
    fc1 = dict(bytes=w1 + T * H * 4 + S * I * 4, flops=2.0 * S * F * H, weight_bytes=w1, used_experts=used)
    fc2 = dict(bytes=w2 + S * I * 4 + S * H * 4, flops=2.0 * S * H * I, weight_bytes=w2, used_experts=used)
    return fc1, fc2


def roofline_for(work, ms, mfma_peak=F16_DENSE_PEAK_TFLOPS):
    intensity = work["flops"] / work["bytes"]
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        ach = work["bytes"] / (ms * 1e-3) / 1e9
        return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4))
    ach = work["flops"] / (ms * 1e-3) / 1e12
    return dict(bound="mfma", achieved=round(ach, 1), peak=mfma_peak, unit="TFLOP/s",
                frac=round(ach / mfma_peak, 4))


def stage_times(qm, call_debug, steps):
    """Average per-stage durations (ms) from HIP events recorded by the library."""
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    evs = []
    for _ in range(6):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e)
    sums = [0.0] * 5
    for _ in range(steps):
        call_debug([e.value for e in evs])
        assert hip.hipEventSynchronize(evs[5]) == 0
        for i in range(5):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[i], evs[i + 1]) == 0
            sums[i] += ms.value
    for e in evs:
        hip.hipEventDestroy(e)
    return dict(zip(("routing", "fc1", "fc1_act", "fc2", "combine"), [s / steps for s in sums]))


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: numpy runs single threaded loops
        return 1


def timed_runs(run, budget_s, max_reps):
    """One untimed warm-up run, then timed runs until about budget_s seconds
    (at least one, at most max_reps): per-run seconds."""
    run()
    ts = []
    t0 = time.perf_counter()
    while len(ts) < max_reps and (not ts or time.perf_counter() - t0 < budget_s):
        t = time.perf_counter()
        run()
        ts.append(time.perf_counter() - t)
    return ts


def cpu_baseline(w, arrs, budget_s=12.0, max_reps=8):
    """Time the float64 oracle on the host cores over a bounded sample of the
    workload (the whole batch for small batches, its first 4 tokens for large
    ones): one warm-up run, then timed runs up to about budget_s seconds;
    tokens/s from the median run."""
    import numpy as np

    import oracle
    attrs = w.attrs()
    ids = list(range(w.tokens)) if w.tokens <= 16 else list(range(4))
    ts = timed_runs(lambda: oracle.qmoe_tokens(ids, *arrs.values(), attrs=attrs), budget_s, max_reps)
    med = float(np.median(ts))
    model, cores = cpu_info()
    if w.tokens <= 16:
        sample = (f"all {w.tokens} tokens of the workload; 1 warm-up run, median of {len(ts)} timed runs "
                  "(every used expert dequantised in float64 once per run)")
    else:
        sample = (f"first 4 tokens of the workload; 1 warm-up run, median of {len(ts)} timed runs "
                  "(their experts dequantised in float64 once per run)")
    return dict(value=round(len(ids) / med, 4), unit="tokens/s", cores=int(_blas_threads()), kind="oracle",
                sample=sample, seconds_per_run=round(med, 3), runs=len(ts), cpu_model=model,
                cores_available=int(cores))


def _sha(path):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


KERNEL_SRC = {
    "qmoe_stream": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "stream.hip"),
    "qmoe_tiled": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "tiled.hip"),
    "qmoe_gemm": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "gemm.hip"),
    "qmoe_gmm_f32": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "gmm.hip"),
    "qmoe_gmm_f32_rows16": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "gmm.hip"),
    "qmoe_gmm_typed": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "gmm_typed.hip"),
    "qmoe_gmm16_rows16": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "gmm_typed.hip"),
    "qmoe_gmm16_tiled": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "gmm_typed.hip"),
    "qmoe_gmm64_rows16": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "gmm_typed.hip"),
    "qmoe_gmm16_stream": os.path.join(ROOT, "quantized_mixture_experts_router_amd", "csrc", "kernels", "gmm_typed.hip"),
}


def gmm_kernel(w):
    """The library's GroupedMatMul kernel for this shape: the weight-streaming
    ones over 16-row tiles when the rows average at most 16 per group (K a
    multiple of 4, N of 4, or of 2 in double; bench tensors are aligned),
    else the LDS-tiled ones (float16 and bfloat16 with K and N multiples of 8
    on the register-transposed kernel)."""
    R = w.M * w.S
    few = R <= 16 * max(1, min(w.G, R))
    rows16 = w.K % 4 == 0 and w.N % 4 == 0 and few
    if w.dtype == "float64":
        return "qmoe_gmm64_rows16" if w.K % 4 == 0 and w.N % 2 == 0 and few else "qmoe_gmm_typed"
    if w.dtype != "float32":
        if rows16:
            return "qmoe_gmm16_stream" if w.K % 8 == 0 and w.N % 8 == 0 else "qmoe_gmm16_rows16"
        return "qmoe_gmm16_tiled" if w.K % 8 == 0 and w.N % 8 == 0 else "qmoe_gmm_typed"
    return "qmoe_gmm_f32_rows16" if rows16 else "qmoe_gmm_f32"


def plan_of(w):
    """The library's launch plan for a workload (qmoe_plan_describe: host
    code, only the shapes are read)."""
    import numpy as np

    import quantized_mixture_experts_router_amd as qm
    from quantized_mixture_experts_router_amd import workloads as W

    s = W.shapes(w)
    names = ("input", "router_probs", "fc1_experts_weights", "fc1_scales", "fc2_experts_weights", "fc2_scales")
    arrs = []
    for n in names:
        dt = np.uint8 if n.endswith("weights") else np.float32
        arrs.append(np.lib.stride_tricks.as_strided(np.zeros(1, dtype=dt), shape=s[n], strides=(0,) * len(s[n])))
    return qm.qmoe_plan_describe(*arrs, w.attrs())


def gemm_kernel(w, which="fc1", plan=None):
    """Kernel the library runs for one GEMM of this workload, read from its
    launch plan (fc1= / fc2= stream, tiled or gemm)."""
    fields = dict(kv.split("=", 1) for kv in (plan or plan_of(w)).split())
    return "qmoe_" + fields[which]


def call_latency(step, n, evict=None):
    """Per-call latency (ms) of n calls timed with events on the launch stream:
    median, p10, p90.  With evict (a large device buffer), it is rewritten
    before every call so that no operand is left in L2 or the Infinity Cache."""
    import numpy as np
    import torch
    ts = []
    for _ in range(n):
        if evict is not None:
            evict.add_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    q = np.percentile(np.array(ts), [50, 10, 90])
    return dict(median=round(float(q[0]), 5), p10=round(float(q[1]), 5), p90=round(float(q[2]), 5), calls=n)


def traffic_for(key, kernel, plan=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel source now in the tree and (for the QMoE GEMMs)
    under the launch plan the library now takes for the workload (K-range
    splits, tile shapes); otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except OSError:
        return None
    ent = rec.get(key)
    if not ent or ent.get("kernel") != kernel:
        return None
    if ent.get("source_sha") != _sha(KERNEL_SRC[kernel]) or launch_fields(ent.get("plan")) != launch_fields(plan):
        return None
    return ent.get("bytes")


def launch_fields(plan):
    """A plan description without its workspace layout (the total size and
    the offset of the segment flag), which moves no HBM bytes."""
    if plan is None:
        return None
    return " ".join(t for t in plan.split() if not t.startswith(("workspace=", "segflag=")))


def copy_calibration(nbytes, reps=3):
    """A plain device-to-device copy of nbytes (for scaling the HBM byte
    counters: its FETCH_SIZE and WRITE_SIZE should each read nbytes)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def gmm_work(w, idx):
    """Algorithmic bytes and FLOPs of one GroupedMatMul call: weights (and
    bias rows) of the groups that receive a row, input rows, output rows, in
    the workload's element type."""
    import numpy as np
    eb = GMM_TYPES[w.dtype][0]
    used = int(np.unique(idx).size)
    wb = used * w.K * w.N * eb + (used * w.N * eb if w.bias else 0)
    return dict(bytes=wb + w.M * w.K * eb + w.M * w.S * w.N * eb, flops=2.0 * w.M * w.S * w.K * w.N,
                weight_bytes=wb, used_groups=used)


def gmm_cpu_baseline(w, a, budget_s=12.0, max_reps=64):
    """The float64 oracle (row-sampled form) on the host cores over the first
    rows of the workload, repeated up to about budget_s seconds."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    rows = list(range(min(4, w.M)))
    done, reps = 0, 0
    t0 = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < budget_s):
        oracle.grouped_matmul_rows(a["input"], a["weights"], a["group_indices"], a["bias"], rows)
        done += len(rows)
        reps += 1
    dt = time.perf_counter() - t0
    model, cores = cpu_info()
    return dict(value=round(done / dt, 4), unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"first {len(rows)} token rows (all {w.S} selections each) x {reps} repetitions",
                seconds=round(dt, 2), cpu_model=model, cores_available=int(cores))


def main_gmm(args):
    """GroupedMatMul on one of its workloads (float32, float16, bfloat16 or
    double): one step = one qmoe_grouped_matmul call (index conversion, group
    permutation, tile GEMM)."""
    import numpy as np
    import torch

    import quantized_mixture_experts_router_amd as qm
    from quantized_mixture_experts_router_amd import workloads as W

    w = W.GMM_WORKLOADS[args.workload]
    a = W.gmm_generate(w)
    torch.cuda.set_device(0)
    tdt = getattr(torch, w.dtype)
    # floating tensors: the float32 draws rounded to the element type
    d = {k: (torch.from_numpy(v).cuda() if v is not None else None) for k, v in a.items()}
    for k in ("input", "weights", "bias"):
        if d[k] is not None:
            d[k] = d[k].to(tdt).contiguous()
    out = torch.empty((w.M, w.S, w.N), dtype=tdt, device="cuda")
    need = qm.qmoe_grouped_matmul_workspace_size(d["input"], d["weights"], d["group_indices"], d["bias"], out)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(events=None):
        qm.qmoe_grouped_matmul(d["input"], d["weights"], d["group_indices"], d["bias"], out, ws, stream, events)

    settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    work = gmm_work(w, a["group_indices"])

    roofline = None
    stages = None
    if not args.no_stage_timing:
        hip = ctypes.CDLL("libamdhip64.so.7")
        evs = []
        for _ in range(3):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e)
        sums = [0.0, 0.0]
        for _ in range(args.steps):
            step([e.value for e in evs])
            assert hip.hipEventSynchronize(evs[2]) == 0
            for i in range(2):
                ms = ctypes.c_float()
                assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[i], evs[i + 1]) == 0
                sums[i] += ms.value
        for e in evs:
            hip.hipEventDestroy(e)
        stages = dict(permutation=sums[0] / args.steps, gemm=sums[1] / args.steps)
        roofline = roofline_for(work, stages["gemm"], GMM_TYPES[w.dtype][1])
        kernel = gmm_kernel(w)
        roofline["kernel"] = kernel
        roofline["avg_ms"] = round(stages["gemm"], 5)
        roofline["algorithmic_bytes"] = int(work["bytes"])
        roofline["algorithmic_flops"] = work["flops"]
        roofline["traffic"] = traffic_for(f"{args.workload}:gemm", kernel)

    cpu = None if args.no_cpu_baseline else gmm_cpu_baseline(w, a)
    line = {
        "metric": f"GroupedMatMul {w.dtype} tokens/s + achieved GB/s or TFLOP/s vs peak",
        "value": round(w.M * args.steps / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": GMM_TYPES[w.dtype][2],
        "data": "synthetic (seeded numpy draws: input N(0,1), weights and bias N(0,1)*wscale, "
                "rounded to the element type; Zipf or uniform distinct group indices)",
        "config": {"workload": w.name, "M": w.M, "K": w.K, "G": w.G, "N": w.N, "S": w.S, "bias": w.bias,
                   "zipf": w.zipf, "element_type": w.dtype},
        "gbs": round(work["bytes"] / (ms_per_step * 1e-3) / 1e9, 1),
        "tflops": round(work["flops"] / (ms_per_step * 1e-3) / 1e12, 2),
        "stage_ms": {k: round(v, 5) for k, v in stages.items()} if stages else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def moe_work(w, counts):
    """Algorithmic bytes and FLOPs of the float MoE projections for one call:
    FC1 (with FC3 when read) and FC2 over the experts that receive a slot."""
    import numpy as np
    used = int(np.count_nonzero(counts))
    T, H, E, I, k, F = w.tokens, w.hidden, w.experts, w.inter, w.k, w.fc1_rows
    S = T * k
    n1 = F + (I if w.fc3 and w.activation in ("silu", "swiglu") else 0)
    b1 = used * n1 * (H + (1 if w.bias else 0)) * 4
    b2 = used * H * (I + (1 if w.bias else 0)) * 4
    fc1 = dict(bytes=b1 + T * H * 4 + S * n1 * 4, flops=2.0 * S * n1 * H, weight_bytes=b1, used_experts=used)
    fc2 = dict(bytes=b2 + S * I * 4 + S * H * 4, flops=2.0 * S * H * I, weight_bytes=b2, used_experts=used)
    return fc1, fc2


def main_moe(args):
    """Float MoE on one of its workloads: one step = one qmoe_moe_forward
    (router, permutation, FC1 (+FC3), activation, FC2, combine)."""
    import numpy as np
    import torch

    import quantized_mixture_experts_router_amd as qm
    from quantized_mixture_experts_router_amd import workloads as W

    w = W.MOE_WORKLOADS[args.workload]
    a = W.moe_generate(w)
    torch.cuda.set_device(0)
    d = {k: torch.from_numpy(v).cuda() for k, v in a.items() if v is not None}
    attrs = qm.make_moe_attrs(w.attrs())
    out = torch.empty_like(d["input"])
    need = qm.qmoe_moe_workspace_size(d, attrs)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(debug=None):
        qm.qmoe_moe_forward(d, attrs, out, ws, stream, debug)

    settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    counts_t = torch.empty(w.experts, dtype=torch.int32, device="cuda")
    step({"counts": counts_t})
    torch.cuda.synchronize()
    fc1_work, fc2_work = moe_work(w, counts_t.cpu().numpy())

    roofline = None
    stages = None
    if not args.no_stage_timing:
        stages = stage_times(qm, lambda events: step({"events": events}), args.steps)
        stages = dict(zip(("routing", "fc1", "activation", "fc2", "combine"), stages.values()))
        key = "fc1" if stages["fc1"] >= stages["fc2"] else "fc2"
        work = fc1_work if key == "fc1" else fc2_work
        roofline = roofline_for(work, stages[key], F32_MATRIX_PEAK_TFLOPS)
        S = w.tokens * w.k
        rows16 = S <= 16 * max(1, min(w.experts, S)) and (w.hidden if key == "fc1" else w.inter) % 4 == 0
        kernel = "qmoe_gmm_f32_rows16" if rows16 else "qmoe_gmm_f32"
        roofline["kernel"] = f"{kernel} ({key.upper()})"
        roofline["avg_ms"] = round(stages[key], 5)
        roofline["algorithmic_bytes"] = int(work["bytes"])
        roofline["algorithmic_flops"] = work["flops"]
        roofline["traffic"] = traffic_for(f"{args.workload}:{key}", kernel)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        except Exception:
            threads = 1
        ids = list(range(min(2, w.tokens)))
        done, reps = 0, 0
        t0 = time.perf_counter()
        args_o = dict(x=a["input"], logits=a["router_probs"], fc1_w=a["fc1_experts_weights"],
                      fc2_w=a["fc2_experts_weights"], fc3_w=a["fc3_experts_weights"], fc1_b=a["fc1_experts_bias"],
                      fc2_b=a["fc2_experts_bias"], fc3_b=a["fc3_experts_bias"])
        while reps < 16 and (reps == 0 or time.perf_counter() - t0 < 12.0):
            oracle.moe_tokens(ids, **args_o, attrs=w.attrs())
            done += len(ids)
            reps += 1
        dt = time.perf_counter() - t0
        model, cores = cpu_info()
        cpu = dict(value=round(done / dt, 4), unit="tokens/s", cores=int(threads), kind="oracle",
                   sample=f"first {len(ids)} tokens x {reps} repetitions (their experts' weights read in float64 "
                          "per token)", seconds=round(dt, 2), cpu_model=model, cores_available=int(cores))

    line = {
        "metric": "float MoE layer tokens/s + achieved GB/s or TFLOP/s vs peak",
        "value": round(w.tokens * args.steps / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy draws: input and logits N(0,1), weights N(0,1)/sqrt(fan-in), "
                "biases N(0,1)*0.1)",
        "config": {"workload": w.name, "tokens": w.tokens, "hidden": w.hidden, "experts": w.experts,
                   "inter": w.inter, "k": w.k, "activation": w.activation, "swiglu_fusion": w.fusion,
                   "bias": w.bias, "fc3": w.fc3, "input_shape": list(w.input_shape)},
        "layer_gbs": round((fc1_work["bytes"] + fc2_work["bytes"]) / (ms_per_step * 1e-3) / 1e9, 1),
        "layer_tflops": round((fc1_work["flops"] + fc2_work["flops"]) / (ms_per_step * 1e-3) / 1e12, 2),
        "stage_ms": {k: round(v, 5) for k, v in stages.items()} if stages else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_info():
    """Host CPU model (from /proc/cpuinfo) and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def settle(step, settle_ms):
    """Run the step back to back for about settle_ms of wall time (untimed),
    so that the GPU reaches its steady clocks before the warm-up steps."""
    import torch
    if settle_ms <= 0:
        return 0
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
    return n


def measure_qmoe(w, steps, warmup, settle_ms, args, arrs=None):
    """Time one QMoE workload: settle, warm-up, K timed steps (one step = one
    qmoe_forward), then per-stage event timing, the roofline of the slower
    GEMM, per-call latency and the oracle's CPU baseline.  Returns a dict of
    the JSON fields."""
    import numpy as np
    import torch

    import quantized_mixture_experts_router_amd as qm
    from quantized_mixture_experts_router_amd import workloads as W

    if arrs is None:
        arrs = W.generate(w)
    torch.cuda.set_device(0)
    d = {k: torch.from_numpy(v).cuda() for k, v in arrs.items()}
    ins = [d[k] for k in ("input", "router_probs", "fc1_experts_weights", "fc1_scales", "fc2_experts_weights",
                          "fc2_scales")]
    attrs = qm.make_attrs(w.attrs())
    out = torch.empty_like(d["input"])
    need = qm.qmoe_workspace_size(*ins, attrs)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        qm.qmoe_forward(*ins, attrs, out, ws, stream)

    settled = settle(step, settle_ms)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / steps
    value = w.tokens * steps / elapsed

    # routing counts (for the algorithmic work of the used experts)
    counts_t = torch.empty(w.held, dtype=torch.int32, device="cuda")  # over the experts the weights hold
    qm.qmoe_forward(*ins, attrs, out, ws, stream, debug={"counts": counts_t})
    torch.cuda.synchronize()
    counts = counts_t.cpu().numpy()
    fc1_work, fc2_work = kernel_work(w, counts)

    roofline = None
    stages = None
    if not args.no_stage_timing:
        def call_debug(events):
            qm.qmoe_forward(*ins, attrs, out, ws, stream, debug={"events": events})
        stages = stage_times(qm, call_debug, steps)
        key = "fc1" if stages["fc1"] >= stages["fc2"] else "fc2"
        work = fc1_work if key == "fc1" else fc2_work
        roofline = roofline_for(work, stages[key])
        plan = qm.qmoe_plan_describe(*ins, attrs)
        kernel = gemm_kernel(w, key, plan)
        roofline["kernel"] = f"{kernel} ({key.upper()})"
        roofline["avg_ms"] = round(stages[key], 5)
        roofline["algorithmic_bytes"] = int(work["bytes"])
        roofline["algorithmic_flops"] = work["flops"]
        roofline["traffic"] = traffic_for(f"{w.name}:{key}", kernel, plan)
        roofline["plan"] = plan

    # Per-call latency outside the throughput loop: warm (operands may sit in
    # L2 / the Infinity Cache from the previous call) and cold (a 1 GiB
    # buffer rewritten before every call).
    latency = None
    if not args.no_latency:
        n = max(10, min(steps, 50))
        evict = torch.empty(1 << 28, dtype=torch.float32, device="cuda").zero_()
        latency = dict(warm=call_latency(step, n), cold=call_latency(step, n, evict))
        del evict

    del ws, d, ins, out
    torch.cuda.empty_cache()
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, arrs)

    total_bytes = fc1_work["bytes"] + fc2_work["bytes"]
    total_flops = fc1_work["flops"] + fc2_work["flops"]
    return {
        "value": round(value, 2),
        "ms_per_step": round(ms_per_step, 5),
        "steps": steps,
        "warmup": warmup,
        "settle_steps": settled,
        "config": dict({"workload": w.name, "tokens": w.tokens, "hidden": w.hidden, "experts": w.experts,
                        "inter": w.inter, "k": w.k, "bits": w.bits, "block_size": w.block_size,
                        "activation": w.activation, "input_shape": list(w.input_shape)},
                       **({"held_experts": w.held, "first_expert": w.first_expert} if w.local_experts else {})),
        "layer_hbm_gbs": round(total_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "layer_hbm_frac": round(total_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_tflops": round(total_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "layer_mfma_frac": round(total_flops / (ms_per_step * 1e-3) / 1e12 / F16_DENSE_PEAK_TFLOPS, 4),
        "stage_ms": {k: round(v, 5) for k, v in stages.items()} if stages else None,
        "roofline": roofline,
        "latency_ms": latency,
        "cpu_baseline": cpu,
    }


def main_crossover(args):
    """Per-step time of one layer's experts (--layer: the decode layer's by
    default) at several token counts (the first T rows of that layer's
    recipe), with the GEMMs forced onto each path (QMOE_PATH = stream |
    tiled) and with the plan's own choice."""
    import dataclasses

    import numpy as np
    import torch

    import quantized_mixture_experts_router_amd as qm
    from quantized_mixture_experts_router_amd import workloads as W

    toks = [int(t) for t in args.crossover.split(",") if t]
    base = W.WORKLOADS[args.layer]
    w = dataclasses.replace(base, name="crossover", input_shape=(max(toks), base.hidden))
    a = W.generate(w)
    torch.cuda.set_device(0)
    d = {k: torch.from_numpy(v).cuda() for k, v in a.items()}
    attrs = qm.make_attrs(w.attrs())
    stream = torch.cuda.current_stream()
    rows = []
    variants = [("stream", {"QMOE_PATH": "stream"}), ("tiled", {"QMOE_PATH": "tiled"}), ("auto", {})]
    if args.tile_rows:
        variants += [(f"stream{r}", {"QMOE_PATH": "stream", "QMOE_STREAM_TILE_ROWS": str(r)})
                     for r in (32, 48, 64)]
    for T in toks:
        ins = [d["input"][:T], d["router_probs"][:T], d["fc1_experts_weights"], d["fc1_scales"],
               d["fc2_experts_weights"], d["fc2_scales"]]
        out = torch.empty_like(ins[0])
        row = {"tokens": T}
        for path, env in variants:
            for key in ("QMOE_PATH", "QMOE_STREAM_TILE_ROWS"):
                os.environ.pop(key, None)
            os.environ.update(env)
            ws = torch.empty(max(qm.qmoe_workspace_size(*ins, attrs), 1), dtype=torch.uint8, device="cuda")

            def step():
                qm.qmoe_forward(*ins, attrs, out, ws, stream)

            settle(step, min(args.settle_ms, 300))
            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                step()
            torch.cuda.synchronize()
            row[f"{path}_ms"] = round((time.perf_counter() - t0) * 1e3 / args.steps, 5)
            del ws
        for key in ("QMOE_PATH", "QMOE_STREAM_TILE_ROWS"):
            os.environ.pop(key, None)
        print(json.dumps(row), file=sys.stderr, flush=True)
        rows.append(row)
    print(json.dumps({"crossover": rows, "layer": f"{base.name} experts (E {base.experts}, H {base.hidden}, "
                      f"I {base.inter}, k {base.k}, int{base.bits}, bs {base.block_size}, "
                      f"{'Zipf' if base.zipf_bias else 'N(0,1)'} logits)",
                      "steps": args.steps, "warmup": args.warmup}), flush=True)


def main():
    args = _args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library runs the layer on one MI355X "
              "(no collectives or sharding across GPUs); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.crossover:
        main_crossover(args)
        return
    if args.workload.startswith("gmm_"):
        main_gmm(args)
        return
    if args.workload.startswith("moe_"):
        main_moe(args)
        return
    from quantized_mixture_experts_router_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    head = measure_qmoe(w, args.steps, args.warmup, args.settle_ms, args)
    line = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 operands (fp32 activations as hi+lo f16 of a power-of-two scaled row), fp32 accumulate",
        "data": "synthetic (seeded numpy draws per workload recipe; weights random uint8)",
        "config": head.pop("config"),
    }
    head.pop("steps")
    head.pop("warmup")
    line.update(head)
    # The metric names int4 decode and prefill: the decode line also carries
    # the prefill layer (same experts, 4096 tokens), timed the same way.
    if args.workload == "decode" and not args.no_prefill:
        pw = W.WORKLOADS["prefill"]
        psteps = args.prefill_steps or max(10, min(args.steps, 40))
        pwarm = max(2, min(args.warmup, 10))
        line["prefill"] = measure_qmoe(pw, psteps, pwarm, args.settle_ms, args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
