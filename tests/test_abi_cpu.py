"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point include/qmoe.h declares, reports the manifest defaults, and its
contract check agrees with the oracle's on every clause."""
import ctypes
import os
import re

import numpy as np
import pytest

import quantized_mixture_experts_router_amd as qm
from oracle import qmoe_oracle as Q
from quantized_mixture_experts_router_amd import workloads as W

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qmoe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qm.LIB_PATH):
        pytest.skip("libqmoe.so not built (run __graft_entry__.build())")
    return qm.library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"qmoe_forward", "qmoe_validate", "qmoe_workspace_size", "qmoe_forward_debug",
            "qmoe_status_string", "qmoe_attrs_default", "qmoe_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_abi_version_and_status_strings(lib):
    assert qm.qmoe_abi_version() == 3
    for s in range(9):
        assert qm.qmoe_status_string(s) != "unknown status"


def test_attribute_defaults_match_manifest(lib):
    a = qm.qmoe_attrs_default()
    # QMoE WebGPU manifest, key "attributes"
    assert a.k == 1 and a.expert_weight_bits == 4 and a.activation_type == 0
    assert a.activation_alpha == 1.0 and a.activation_beta == 0.0
    assert a.normalize_routing_weights == 0 and a.swiglu_fusion == 0
    assert a.use_sparse_mixer == 0 and a.weights_prepacked == -1 and a.quant_type == 0
    assert a.block_size == 0 and a.routing == 0
    assert a.has_swiglu_limit == 0  # swiglu_limit is optional: omitted means no clamp
    assert a.first_expert == 0  # the weights hold every expert from expert 0


KIND = {"shape": 2, "attr": 3, "unsupported": 4, "dtype": 7}


def _case(rng, **kw):
    base = dict(tokens_shape=(6,), hidden=32, experts=4, inter=32, k=1, bits=4, block_size=0,
                activation="relu")
    base.update(kw)
    return W.random_case(rng, **base)


def _mutate(a, attrs, mut):
    if mut == "blocks64":
        attrs["block_size"] = 64
        a["fc1_scales"] = a["fc1_scales"][..., None]
        a["fc2_scales"] = a["fc2_scales"][..., None]
    elif mut == "router_rows":
        a["router_probs"] = a["router_probs"][:-1]
    elif mut == "fc2_rows":
        a["fc2_experts_weights"] = a["fc2_experts_weights"][:, :-1]
    elif mut == "packed_cols":
        a["fc1_experts_weights"] = a["fc1_experts_weights"][:, :, :-1]
    elif mut == "scale_rank":
        a["fc1_scales"] = a["fc1_scales"][..., None]
    elif mut == "dtype":
        a["input"] = a["input"].astype(np.float64)
    elif mut == "rank4":
        a["input"] = a["input"][None, None]
    elif mut == "share_more":
        a["router_probs"] = a["router_probs"][:, :3]   # weights hold 4 experts, router only 3
    elif mut.startswith("share"):
        # weights for experts [first, first + held) of the router's 4
        first, held = {"share": (1, 2), "share_top": (2, 2), "share_none": (4, 0), "share_past": (3, 2),
                       "share_neg": (-1, 2)}[mut]
        attrs["first_expert"] = first
        for n in ("fc1_experts_weights", "fc1_scales", "fc2_experts_weights", "fc2_scales"):
            a[n] = a[n][max(first, 0):max(first, 0) + held]


CASES = [
    ("ok", {}, None), ("k0", dict(k=0), None), ("k_gt_e", dict(k=5), None),
    ("bits2", dict(expert_weight_bits=2), None), ("normalize2", dict(normalize_routing_weights=2), None),
    ("prepacked1", dict(weights_prepacked=1), None), ("prepacked2", dict(weights_prepacked=2), None),
    ("sparse", dict(use_sparse_mixer=1), None), ("quant_fp", dict(quant_type="fp"), None),
    ("relu_fused", dict(swiglu_fusion=1), None), ("fusion2", dict(swiglu_fusion=2), None),
    ("bs8", dict(block_size=8), None), ("bs24", dict(block_size=24), None),
    ("bs64_not_dividing", {}, "blocks64"), ("router_rows", {}, "router_rows"), ("fc2_rows", {}, "fc2_rows"),
    ("packed_cols", {}, "packed_cols"), ("scale_rank", {}, "scale_rank"), ("dtype", {}, "dtype"),
    ("rank4", {}, "rank4"), ("moe_norm", dict(routing="moe", normalize_routing_weights=1), None),
    ("bs16", dict(block_size=16), "bs16"), ("swiglu", dict(activation_type="swiglu", swiglu_fusion=1), "swiglu"),
    ("share", {}, "share"), ("share_top", {}, "share_top"), ("share_none", {}, "share_none"),
    ("share_past", {}, "share_past"), ("share_neg", {}, "share_neg"), ("share_more", {}, "share_more"),
]


@pytest.mark.parametrize("name,over,mut", CASES, ids=[c[0] for c in CASES])
def test_validate_agrees_with_oracle(lib, name, over, mut):
    rng = np.random.default_rng(7)
    if mut == "bs16":
        w, a = _case(rng, block_size=16)
    elif mut == "swiglu":
        w, a = _case(rng, activation="swiglu")
    else:
        w, a = _case(rng)
    attrs = dict(w.attrs(), **over)
    if mut not in (None, "bs16", "swiglu"):
        _mutate(a, attrs, mut)
    try:
        Q.validate(*a.values(), attrs=attrs)
        expect = 0
    except Q.ContractError as e:
        expect = KIND[e.kind]
    got = qm.qmoe_validate(*a.values(), attrs=attrs)
    assert got == expect, (name, got, expect)


def test_validate_output_shape_and_zero_sizes(lib):
    rng = np.random.default_rng(8)
    w, a = _case(rng)
    out_bad = np.zeros((5, 32), dtype=np.float32)
    assert qm.qmoe_validate(*a.values(), output=out_bad, attrs=w.attrs()) == 2
    assert qm.qmoe_validate(*a.values(), output=a["input"], attrs=w.attrs()) == 0
    # T == 0 and I == 0 are in contract
    b = dict(a, input=a["input"][:0], router_probs=a["router_probs"][:0])
    assert qm.qmoe_validate(*b.values(), attrs=w.attrs()) == 0
    assert qm.qmoe_workspace_size(*b.values(), attrs=w.attrs()) == 0
    w0, c = _case(rng, inter=0)
    assert qm.qmoe_validate(*c.values(), attrs=w0.attrs()) == 0


def test_workspace_size_covers_intermediates(lib):
    for name in ("decode", "prefill", "fine", "large_e"):
        w = W.WORKLOADS[name]
        s = W.shapes(w)
        fake = {k: np.lib.stride_tricks.as_strided(np.zeros(1, dtype=np.float32 if "weights" not in k else np.uint8),
                                                    shape=v, strides=(0,) * len(v)) for k, v in s.items()}
        n = qm.qmoe_workspace_size(fake["input"], fake["router_probs"], fake["fc1_experts_weights"],
                                   fake["fc1_scales"], fake["fc2_experts_weights"], fake["fc2_scales"], w.attrs())
        S = w.tokens * w.k
        assert n >= 4 * S * w.hidden + 4 * S * w.inter + 4 * w.tokens * w.hidden
        # plus split-K partials on the weight-streaming path (a few MB at decode sizes)
        assert n < 3 * (4 * S * w.hidden + 4 * S * w.inter + 4 * w.tokens * w.hidden) + (64 << 20)


def test_null_arguments(lib):
    assert lib.qmoe_validate(None, None, None, None, None, None, None, None) == 1
    a = qm.qmoe_attrs_default()
    assert lib.qmoe_workspace_size(None, None, None, None, None, None, ctypes.byref(a), None) == 1


# ---------------------------------------------------------------- GroupedMatMul
def _gmm(M=4, K=3, G=2, N=5, S=2, dt=np.float32, it=np.int64, bias=True):
    z = lambda shape, d: np.lib.stride_tricks.as_strided(np.zeros(1, dtype=d), shape=shape,
                                                         strides=(0,) * len(shape))
    return dict(input=z((M, K), dt), weights=z((G, K, N), dt), group_indices=z((M, S), it),
                bias=z((G, N), dt) if bias else None, output=z((M, S, N), dt))


def _gmm_status(**kw):
    try:
        qm.qmoe_grouped_matmul_workspace_size(**kw)
        return 0
    except qm.QmoeError as e:
        return e.status


def test_grouped_matmul_contract(lib):
    # ONNX "GroupedMatMul - 29": Inputs, Outputs, Type Constraints
    assert _gmm_status(**_gmm()) == 0
    assert _gmm_status(**_gmm(it=np.int32, bias=False)) == 0
    assert _gmm_status(**dict(_gmm(), output=None)) == 0
    # shape clauses
    a = _gmm()
    assert _gmm_status(**dict(a, input=a["input"][:, :2])) == 2               # K mismatch
    assert _gmm_status(**dict(a, group_indices=a["group_indices"][:3])) == 2  # M mismatch
    assert _gmm_status(**dict(a, bias=a["bias"][:1])) == 2                    # bias [G, N]
    assert _gmm_status(**dict(a, output=a["output"][:, :1])) == 2             # output [M, S, N]
    assert _gmm_status(**dict(a, input=a["input"][None])) == 2                # rank 3 input
    # dtype clauses: T is one float type for input, weights, bias, output
    assert _gmm_status(**_gmm(it=np.int16)) == 7
    assert _gmm_status(**_gmm(it=np.float32)) == 7
    assert _gmm_status(**dict(a, weights=a["weights"].astype(np.float64))) == 7
    assert _gmm_status(**_gmm(dt=np.uint8)) == 7
    for dt in (np.float16, np.float64):  # the page's other types: accepted
        assert _gmm_status(**_gmm(dt=dt)) == 0
        b = _gmm(dt=dt)
        assert _gmm_status(**dict(b, bias=b["bias"].astype(np.float32))) == 7   # one T for all four
    # group count limit of the permutation (G + 1 buckets <= 1024)
    assert _gmm_status(**_gmm(G=1023)) == 0
    assert _gmm_status(**_gmm(G=1024)) == 4


def test_grouped_matmul_workspace_and_empty(lib):
    # empty outputs need no workspace; G == 0 and K == 0 are in contract
    for kw in (dict(M=0), dict(S=0), dict(N=0)):
        assert qm.qmoe_grouped_matmul_workspace_size(**_gmm(**kw)) == 0
    for kw in (dict(G=0), dict(K=0)):
        assert qm.qmoe_grouped_matmul_workspace_size(**_gmm(**kw)) > 0
    # index copy, permutation and tile table grow with M * S
    small = qm.qmoe_grouped_matmul_workspace_size(**_gmm(M=64, S=2))
    big = qm.qmoe_grouped_matmul_workspace_size(**_gmm(M=4096, S=8))
    assert big >= 2 * 4 * 4096 * 8 > small


def test_grouped_matmul_null_arguments(lib):
    n = ctypes.c_size_t(0)
    assert lib.qmoe_grouped_matmul_workspace_size(None, None, None, None, None, ctypes.byref(n)) == 1
    a = {k: qm.describe(v, False) for k, v in _gmm().items()}
    refs = [ctypes.byref(a[k]) for k in ("input", "weights", "group_indices", "bias", "output")]
    assert lib.qmoe_grouped_matmul_workspace_size(*refs, None) == 1
    # missing output descriptor, then a missing device pointer
    assert lib.qmoe_grouped_matmul(*refs[:4], None, None, 0, None) == 1
    assert lib.qmoe_grouped_matmul(*refs, None, 1 << 20, None) == 1


# ---------------------------------------------------------------- float MoE
def test_moe_attribute_defaults_match_readme(lib):
    a = qm.qmoe_moe_attrs_default()
    # MoE README, Attributes table
    assert a.k == 1 and a.activation_type == 0 and a.swiglu_fusion == 0
    assert a.activation_alpha == 1.0 and a.activation_beta == 0.0
    assert a.normalize_routing_weights == 0 and a.use_sparse_mixer == 0


def _moe_tensors(a):
    return {"input": a["x"], "router_probs": a["logits"], "fc1_experts_weights": a["fc1_w"],
            "fc1_experts_bias": a["fc1_b"], "fc2_experts_weights": a["fc2_w"], "fc2_experts_bias": a["fc2_b"],
            "fc3_experts_weights": a["fc3_w"], "fc3_experts_bias": a["fc3_b"]}


def test_moe_validate_agrees_with_oracle(lib):
    from test_oracle_moe import CONTRACT, _case
    from oracle import moe_oracle as MO
    for name, mut, over, kind in CONTRACT:
        rng = np.random.default_rng(9)
        a, attrs = _case(rng)
        mut(a)
        attrs = dict(attrs, **over)
        with pytest.raises(Q.ContractError) as ei:
            MO.moe_validate(**a, attrs=attrs)
        assert ei.value.kind == kind
        assert qm.qmoe_moe_validate(_moe_tensors(a), attrs) == KIND[kind], name
    # accepted combinations, including unused FC3 and both fused layouts
    rng = np.random.default_rng(10)
    for act, fusion, fc3 in [("relu", 2, True), ("gelu", 0, True), ("swiglu", 1, False), ("swiglu", 2, False),
                             ("swiglu", 0, True), ("silu", 0, False), ("identity", 1, False)]:
        a, attrs = _case(rng, act=act, fusion=fusion, fc3=fc3)
        MO.moe_validate(**a, attrs=attrs)
        assert qm.qmoe_moe_validate(_moe_tensors(a), attrs, output=a["x"]) == 0, (act, fusion, fc3)


def test_moe_dtype_output_and_empty(lib):
    from test_oracle_moe import _case
    rng = np.random.default_rng(11)
    a, attrs = _case(rng)
    t = _moe_tensors(a)
    assert qm.qmoe_moe_validate(dict(t, fc2_experts_bias=t["fc2_experts_bias"].astype(np.float64)), attrs) == 7
    assert qm.qmoe_moe_validate(t, attrs, output=np.zeros((5, 7), np.float32)) == 2
    # T == 0 and H == 0 need no workspace; I == 0 is in contract
    a0, attrs0 = _case(rng, T=0)
    assert qm.qmoe_moe_workspace_size(_moe_tensors(a0), attrs0) == 0
    aI, attrsI = _case(rng, I=0)
    assert qm.qmoe_moe_validate(_moe_tensors(aI), attrsI) == 0
    assert qm.qmoe_moe_workspace_size(_moe_tensors(aI), attrsI) > 0
    # E above the routing kernels' limit
    aE, attrsE = _case(rng, E=1025, T=2, H=4, I=4)
    assert qm.qmoe_moe_validate(_moe_tensors(aE), attrsE) == 4


def test_moe_null_arguments(lib):
    a = qm.qmoe_moe_attrs_default()
    assert lib.qmoe_moe_validate(*([None] * 9), ctypes.byref(a)) == 1
    n = ctypes.c_size_t(0)
    assert lib.qmoe_moe_workspace_size(*([None] * 8), ctypes.byref(a), ctypes.byref(n)) == 1


def test_swiglu_limit_contract_agrees_with_oracle(lib):
    rng = np.random.default_rng(12)
    w, a = W.random_case(rng, tokens_shape=(3,), hidden=32, experts=4, inter=32, k=2, bits=4, block_size=0,
                         activation="swiglu")
    for lim, kind in ((0.0, "attr"), (-2.0, "attr"), (float("nan"), "attr"), (3.5, None), (None, None)):
        attrs = dict(w.attrs(), swiglu_limit=lim)
        if kind:
            with pytest.raises(Q.ContractError):
                Q.validate(*a.values(), attrs=attrs)
        else:
            Q.validate(*a.values(), attrs=attrs)
        assert qm.qmoe_validate(*a.values(), attrs=attrs) == (KIND[kind] if kind else 0), lim
    from test_oracle_moe import _case
    from oracle import moe_oracle as MO
    am, attrs_m = _case(rng, act="swiglu", fusion=1)
    for lim, code in ((0.0, 3), (float("nan"), 3), (1.5, 0)):
        assert qm.qmoe_moe_validate(_moe_tensors(am), dict(attrs_m, swiglu_limit=lim)) == code
    a2 = qm.make_attrs(dict(swiglu_limit=2.5))
    assert a2.has_swiglu_limit == 1 and a2.swiglu_limit == 2.5
    assert qm.make_attrs(dict(swiglu_limit=None)).has_swiglu_limit == 0
