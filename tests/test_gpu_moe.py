"""GPU parity of the float MoE operator (com.microsoft.MoE README) through the
C ABI against the float64 oracle.

Bar (stated before the kernels ran): top-k indices, counts, offsets and the
permutation bit-exact; routing weights within 1e-6; every output element
within 1e-4 x RMS of the oracle's output.  The arithmetic is float32
throughout (two chained dot products of length H and I, float32 libm in the
activation): rounding grows like 2^-24 sqrt(H + I) relative to the output
scale, under 1e-5 at the largest sizes here, so 1e-4 leaves a tenfold margin
while a wrong or missing term (of order 1/sqrt(H) of the output) fails it.
Small cases compare every element; full-size workloads compare the routing
of every token and sampled output rows the oracle computes one by one.
"""
import numpy as np
import pytest

import oracle
import quantized_mixture_experts_router_amd as qm
from quantized_mixture_experts_router_amd import workloads as W

from gpu_util import say

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-4
W_TOL = 1e-6


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _run(torch, arrs, attrs, label):
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in arrs.items() if v is not None}
    x = d["input"]
    T = int(np.prod(arrs["input"].shape[:-1]))
    E = arrs["router_probs"].shape[1]
    k = attrs["k"]
    dbg = dict(topk_idx=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
               topk_w=torch.full((T * k,), -7.0, dtype=torch.float32, device="cuda"),
               counts=torch.full((E,), -7, dtype=torch.int32, device="cuda"),
               offsets=torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
               perm=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"))
    out = torch.full_like(x, float("nan"))
    need = qm.qmoe_moe_workspace_size(d, attrs)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")  # NaN floats
    say(f"[moe] {label} x={tuple(x.shape)} E={E} I={arrs['fc2_experts_weights'].shape[2]} attrs={attrs} "
        f"fc3={arrs.get('fc3_experts_weights') is not None} ws={need}")
    qm.moe_forward(d, attrs, output=out, workspace=ws, debug=dbg if T > 0 else None)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy()}
    res.update({kk: v.cpu().numpy() for kk, v in dbg.items()})
    return res


def _args(arrs):
    return dict(x=arrs["input"], logits=arrs["router_probs"], fc1_w=arrs["fc1_experts_weights"],
                fc2_w=arrs["fc2_experts_weights"], fc3_w=arrs.get("fc3_experts_weights"),
                fc1_b=arrs.get("fc1_experts_bias"), fc2_b=arrs.get("fc2_experts_bias"),
                fc3_b=arrs.get("fc3_experts_bias"))


def _check_routing(res, inter, T, k):
    np.testing.assert_array_equal(res["topk_idx"].reshape(T, k), inter["sel"])
    err = np.abs(res["topk_w"].reshape(T, k).astype(np.float64) - inter["w"])
    assert np.all(err <= W_TOL * np.maximum(1.0, np.abs(inter["w"]))), float(err.max())
    np.testing.assert_array_equal(res["counts"], inter["counts"])
    np.testing.assert_array_equal(res["offsets"], inter["offsets"])
    np.testing.assert_array_equal(res["perm"], inter["perm"])


def _check_out(got, ref, label):
    ref = np.asarray(ref, dtype=np.float64)
    assert not np.isnan(got).any(), f"{label}: unwritten output"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.abs(got.astype(np.float64) - ref).max()) if ref.size else 0.0
    say(f"[moe] {label} max err {err:.3g} rms {rms:.3g} ratio {err / max(rms, 1e-300):.3g}")
    assert err <= OUT_TOL * rms, f"{label}: max err {err} > {OUT_TOL} x rms {rms}"


def _full(torch, w, arrs, label):
    attrs = w.attrs()
    res = _run(torch, arrs, attrs, label)
    ref, inter = oracle.moe(**_args(arrs), attrs=attrs, return_intermediates=True)
    _check_routing(res, inter, w.tokens, w.k)
    _check_out(res["out"], ref, label)


ACT_CASES = [  # activation, fusion, fc3
    ("relu", 0, False), ("gelu", 0, False), ("identity", 0, False), ("silu", 0, False), ("silu", 0, True),
    ("swiglu", 0, True), ("swiglu", 1, False), ("swiglu", 2, False),
    ("relu", 0, True),  # FC3 given but not read
]
SIZES = [  # tokens shape, hidden, experts, inter, k: 16-row tiles, then 64-row tiles
    ((6,), 64, 8, 96, 2),
    ((3, 70), 128, 4, 160, 2),
]


@pytest.mark.parametrize("size", SIZES, ids=["tiles16", "tiles64"])
@pytest.mark.parametrize("act,fusion,fc3", ACT_CASES, ids=[f"{a}{f}{'+fc3' if c else ''}" for a, f, c in ACT_CASES])
def test_activations_and_layouts(torch, act, fusion, fc3, size):
    rng = np.random.default_rng(1000 + 10 * ACT_CASES.index((act, fusion, fc3)) + SIZES.index(size))
    shape, H, E, I, k = size
    for bias in (True, False):
        w, a = W.moe_random_case(rng, tokens_shape=shape, hidden=H, experts=E, inter=I, k=k, activation=act,
                                 fusion=fusion, bias=bias, fc3=fc3)
        _full(torch, w, a, f"{act}{fusion} fc3={fc3} bias={bias} {shape}")


@pytest.mark.parametrize("alpha,beta,normalize", [(1.702, 1.0, 0), (0.5, -0.25, 1)])
def test_swiglu_alpha_beta_and_normalised_routing(torch, alpha, beta, normalize):
    rng = np.random.default_rng(21)
    for fusion, fc3 in ((0, True), (1, False), (2, False)):
        w, a = W.moe_random_case(rng, tokens_shape=(20,), hidden=96, experts=6, inter=64, k=3, activation="swiglu",
                                 fusion=fusion, fc3=fc3, normalize=normalize, alpha=alpha, beta=beta)
        _full(torch, w, a, f"swiglu{fusion} a={alpha} b={beta} n={normalize}")


@pytest.mark.parametrize("fusion,fc3", [(0, True), (1, False), (2, False)])
def test_swiglu_limit(torch, fusion, fc3):
    rng = np.random.default_rng(30 + fusion)
    for shape in ((6,), (3, 70)):  # 16-row and 64-row tiles
        w, a = W.moe_random_case(rng, tokens_shape=shape, hidden=96, experts=4, inter=64, k=2,
                                 activation="swiglu", fusion=fusion, fc3=fc3, alpha=1.702, beta=1.0)
        for lim in (0.1, 0.5):
            attrs = dict(w.attrs(), swiglu_limit=lim)
            res = _run(torch, a, attrs, f"limit={lim}")
            ref, inter = oracle.moe(**_args(a), attrs=attrs, return_intermediates=True)
            _check_routing(res, inter, w.tokens, w.k)
            _check_out(res["out"], ref, f"swiglu{fusion} limit={lim} {shape}")


@pytest.mark.parametrize("case", [
    dict(tokens_shape=(7,), hidden=30, experts=3, inter=18, k=2, activation="gelu"),     # H, I not multiples of 4
    dict(tokens_shape=(9,), hidden=64, experts=5, inter=20, k=1, activation="silu", fc3=True),
    dict(tokens_shape=(4,), hidden=32, experts=4, inter=16, k=4, activation="relu"),     # k == E
    dict(tokens_shape=(64,), hidden=128, experts=128, inter=64, k=8, activation="swiglu", fusion=1,
         logit_sigma=1.5),                                                                # many experts
    dict(tokens_shape=(300,), hidden=64, experts=16, inter=48, k=4, activation="identity"),  # S > 1024
    dict(tokens_shape=(2, 3), hidden=16, experts=4, inter=8, k=2, activation="relu"),     # rank-3 input
], ids=["unaligned", "k1-silu-fc3", "k-eq-E", "E128", "S1200", "rank3"])
def test_shapes_and_front_ends(torch, case):
    rng = np.random.default_rng(22)
    w, a = W.moe_random_case(rng, **case)
    _full(torch, w, a, f"{case}")


def test_streaming_fc1_one_strip_per_wavefront(torch):
    # FC1 wide enough for one column strip per wavefront (no K split), with
    # a K tail (H % 32 != 0); FC2 narrow (K split)
    rng = np.random.default_rng(26)
    w, a = W.moe_random_case(rng, tokens_shape=(8,), hidden=68, experts=8, inter=16400, k=2, activation="relu")
    _full(torch, w, a, "fc1-strips")


def test_zero_inter_gives_weighted_fc2_bias(torch):
    rng = np.random.default_rng(23)
    w, a = W.moe_random_case(rng, tokens_shape=(10,), hidden=32, experts=4, inter=0, k=2, activation="relu")
    _full(torch, w, a, "I=0")


def test_zero_tokens_is_a_no_op(torch):
    rng = np.random.default_rng(24)
    w, a = W.moe_random_case(rng, tokens_shape=(0,), hidden=32, experts=4, inter=16, k=2, activation="relu")
    res = _run(torch, a, w.attrs(), "T=0")
    assert res["out"].shape == (0, 32)


@pytest.mark.parametrize("name", sorted(W.MOE_WORKLOADS))
def test_full_size_workloads_sampled(torch, name):
    w = W.MOE_WORKLOADS[name]
    a = W.moe_generate(w)
    attrs = w.attrs()
    res = _run(torch, a, attrs, name)
    # routing of every token, exactly
    sel, wts = oracle.route(a["router_probs"], w.k, "moe", w.normalize)
    counts, offsets, perm = oracle.expert_permutation(sel, w.experts)
    _check_routing(res, dict(sel=sel, w=wts, counts=counts, offsets=offsets, perm=perm), w.tokens, w.k)
    # sampled output rows against the oracle (each row re-reads its experts'
    # weights in float64, so a few rows)
    rng = np.random.default_rng(25)
    rows = sorted(set([0, w.tokens - 1]) | set(rng.choice(w.tokens, size=2, replace=False).tolist()))
    ref = oracle.moe_tokens(rows, **_args(a), attrs=attrs)
    got = res["out"].reshape(w.tokens, w.hidden)[rows]
    _check_out(got, ref, f"{name} rows {rows}")
    assert np.isfinite(res["out"]).all()
