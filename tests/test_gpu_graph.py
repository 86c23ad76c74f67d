"""The operators inside a captured HIP graph (torch.cuda.CUDAGraph).

qmoe_forward, qmoe_grouped_matmul and qmoe_moe_forward only enqueue kernels
on the caller's stream (no allocation, no synchronisation, no memset nodes),
so one call can be captured and replayed.  Each case captures one call, then
replays the graph several times with eager work and a synchronisation between
replays and new values written into the captured input buffers before some of
them, and checks every replay bit for bit against an eager call on the same
inputs (the kernels sum in a fixed order, so the two agree exactly), and the
first eager call against the oracle.
"""
import numpy as np
import pytest

import oracle
from oracle import moe_oracle as MOE
from quantized_mixture_experts_router_amd import workloads as W
import quantized_mixture_experts_router_amd as qm

from gpu_util import check_output, say

pytestmark = pytest.mark.gpu

NAMES = ("input", "router_probs", "fc1_experts_weights", "fc1_scales", "fc2_experts_weights", "fc2_scales")


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _replays(torch, enqueue, out_g, out_e, ws, mutate, label, n=5):
    """Capture enqueue(out_g, stream) and replay it n times; before replays 2
    and 4 mutate() writes new inputs.  Returns the first eager result."""
    def eager():
        enqueue(out_e, torch.cuda.current_stream())
        torch.cuda.synchronize()
        return out_e.cpu().numpy()

    first = ref = eager()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enqueue(out_g, side)  # warm-up off the default stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue(out_g, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(n):
        if r in (2, 4):
            mutate()
            torch.cuda.synchronize()
            ref = eager()
        out_g.fill_(float("nan"))
        ws.fill_(0xFF)
        g.replay()
        torch.cuda.synchronize()
        got = out_g.cpu().numpy()
        assert np.array_equal(got, ref), f"{label}: replay {r} differs from the eager call"
        assert np.array_equal(eager(), ref)  # eager work on the same buffers between replays
    say(f"  {label}: {n} replays bit-identical to eager calls")
    return first


@pytest.mark.parametrize("case", [
    # (T, H, E, I, k, bits, bs, act)
    (16, 2048, 8, 1024, 2, 4, 64, "swiglu"),   # weight streaming, K-range partials
    (200, 256, 6, 192, 2, 4, 32, "swiglu"),    # LDS-tiled GEMMs
    (70, 136, 5, 96, 3, 8, 0, "relu"),         # register-tiled GEMMs
])
def test_qmoe_forward_replayed_from_a_graph(torch, case):
    T, H, E, I, k, bits, bs, act = case
    say(f"[case] graph qmoe T={T} H={H} E={E} I={I} k={k} bits={bits} bs={bs} {act}")
    rng = np.random.default_rng(4000 + T)
    w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, bits=bits, block_size=bs,
                         activation=act)
    attrs = w.attrs()
    dev = {n: torch.from_numpy(np.ascontiguousarray(a[n])).cuda() for n in NAMES}
    args = [dev[n] for n in NAMES]
    ws = torch.empty(max(qm.qmoe_workspace_size(*args, attrs), 1), dtype=torch.uint8, device="cuda")
    out_g, out_e = torch.empty_like(dev["input"]), torch.empty_like(dev["input"])

    def mutate():
        dev["input"].copy_(torch.from_numpy(rng.standard_normal(a["input"].shape).astype(np.float32)))
        dev["router_probs"].copy_(torch.from_numpy(rng.standard_normal(a["router_probs"].shape).astype(np.float32)))

    first = _replays(torch, lambda out, st: qm.qmoe_forward(*args, attrs, out, ws, st), out_g, out_e, ws, mutate,
                     f"qmoe T{T}")
    check_output(first, oracle.qmoe(*[a[n] for n in NAMES], attrs=attrs), f"qmoe T{T} eager")


@pytest.mark.parametrize("case", [
    # (M, K, G, N, S, bias)
    (16, 512, 8, 1024, 2, True),    # 16-row weight streaming
    (300, 256, 5, 384, 3, False),   # LDS-tiled
])
def test_grouped_matmul_replayed_from_a_graph(torch, case):
    M, K, G, N, S, bias = case
    say(f"[case] graph GroupedMatMul M={M} K={K} G={G} N={N} S={S} bias={bias}")
    w = W.GmmWorkload("graph", M, K, G, N, S, bias=bias)
    a = W.gmm_generate(w, seed=5000 + M, index_dtype=np.int32)
    rng = np.random.default_rng(5100 + M)
    dx = torch.from_numpy(a["input"]).cuda()
    dw = torch.from_numpy(a["weights"]).cuda()
    di = torch.from_numpy(a["group_indices"]).cuda()
    db = torch.from_numpy(a["bias"]).cuda() if bias else None
    out_g = torch.empty((M, S, N), dtype=torch.float32, device="cuda")
    out_e = torch.empty_like(out_g)
    need = qm.qmoe_grouped_matmul_workspace_size(dx, dw, di, db, out_g)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def mutate():
        dx.copy_(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)))
        di.copy_(torch.from_numpy(rng.integers(0, G, size=(M, S)).astype(np.int32)))

    first = _replays(torch, lambda out, st: qm.qmoe_grouped_matmul(dx, dw, di, db, out, ws, st), out_g, out_e, ws,
                     mutate, f"GroupedMatMul M{M}")
    ref = oracle.grouped_matmul_rows(a["input"], a["weights"], a["group_indices"], a["bias"] if bias else None)
    check_output(first, ref, f"GroupedMatMul M{M} eager")


@pytest.mark.parametrize("case", [
    # (T, H, E, I, k, act, fusion)
    (12, 512, 8, 256, 2, "swiglu", 1),   # 16-row weight streaming
    (150, 128, 4, 96, 2, "gelu", 0),     # LDS-tiled
])
def test_moe_forward_replayed_from_a_graph(torch, case):
    T, H, E, I, k, act, fusion = case
    say(f"[case] graph MoE T={T} H={H} E={E} I={I} k={k} {act}")
    rng = np.random.default_rng(6000 + T)
    w, a = W.moe_random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, activation=act,
                             fusion=fusion)
    attrs = w.attrs()
    d = {n: torch.from_numpy(np.ascontiguousarray(v)).cuda() for n, v in a.items() if v is not None}
    out_g, out_e = torch.empty_like(d["input"]), torch.empty_like(d["input"])
    ws = torch.empty(max(qm.qmoe_moe_workspace_size(d, attrs), 1), dtype=torch.uint8, device="cuda")

    def mutate():
        d["input"].copy_(torch.from_numpy(rng.standard_normal(a["input"].shape).astype(np.float32)))
        d["router_probs"].copy_(torch.from_numpy(rng.standard_normal(a["router_probs"].shape).astype(np.float32)))

    first = _replays(torch, lambda out, st: qm.qmoe_moe_forward(d, attrs, out, ws, st), out_g, out_e, ws, mutate,
                     f"MoE T{T}")
    ref = MOE.moe(a["input"], a["router_probs"], a["fc1_experts_weights"], a["fc2_experts_weights"],
                  a.get("fc3_experts_weights"), a.get("fc1_experts_bias"), a.get("fc2_experts_bias"),
                  a.get("fc3_experts_bias"), attrs=attrs)
    check_output(first, ref, f"MoE T{T} eager")
