"""Pins of the float MoE oracle (com.microsoft.MoE README) against values and
identities fixed outside it: textbook GELU / SiLU values and library
routines, the equivalence of the three SwiGLU operand layouts, the QMoE
oracle on dequantised weights (MoE routing mode), a composed-matrix closed
form for the identity activation, the fc2-bias-before-weight closed form,
and the contract clauses of the Inputs and Attributes tables."""
import math

import numpy as np
import pytest
import scipy.special as sp

from oracle import moe_oracle as M
from oracle import qmoe_oracle as Q


def _case(rng, T=5, H=8, E=4, I=6, act="relu", fusion=0, fc3=False, bias=True, k=2, lead=None):
    F = 2 * I if act == "swiglu" and fusion in (1, 2) else I
    x = rng.standard_normal(lead + (H,) if lead else (T, H)).astype(np.float32)
    T = int(np.prod(x.shape[:-1]))
    a = dict(x=x, logits=rng.standard_normal((T, E)).astype(np.float32),
             fc1_w=(0.3 * rng.standard_normal((E, F, H))).astype(np.float32),
             fc2_w=(0.3 * rng.standard_normal((E, H, I))).astype(np.float32),
             fc3_w=(0.3 * rng.standard_normal((E, I, H))).astype(np.float32) if fc3 else None,
             fc1_b=(0.1 * rng.standard_normal((E, F))).astype(np.float32) if bias else None,
             fc2_b=(0.1 * rng.standard_normal((E, H))).astype(np.float32) if bias else None,
             fc3_b=(0.1 * rng.standard_normal((E, I))).astype(np.float32) if bias and fc3 else None)
    attrs = dict(k=k, activation_type=act, swiglu_fusion=fusion)
    return a, attrs


# ---------------------------------------------------------------- activations
def test_gelu_textbook_values_and_library_cdf():
    # GELU(h) = h Phi(h): Phi(1) = 0.8413447460685429 (standard normal table)
    assert M.gelu(1.0) == pytest.approx(0.8413447460685429, abs=1e-15)
    assert M.gelu(-1.0) == pytest.approx(-0.15865525393145707, abs=1e-15)
    assert M.gelu(0.0) == 0.0
    h = np.linspace(-6, 6, 97)
    np.testing.assert_allclose(M.gelu(h), h * sp.ndtr(h), rtol=1e-14, atol=1e-300)
    # odd part is the identity: GELU(h) - GELU(-h) = h
    np.testing.assert_allclose(M.gelu(h) - M.gelu(-h), h, rtol=1e-13, atol=1e-14)


def test_silu_values():
    assert M.moe_activation(np.array([1.0]), "silu")[0] == pytest.approx(0.7310585786300049, abs=1e-15)
    h = np.linspace(-8, 8, 65)
    np.testing.assert_allclose(M.moe_activation(h, "silu"), h * sp.expit(h), rtol=1e-14, atol=1e-300)
    u = np.linspace(2, -2, 65)
    np.testing.assert_allclose(M.moe_activation(h, "silu", u3=u), h * sp.expit(h) * u, rtol=1e-14, atol=1e-300)


def test_relu_identity_values():
    h = np.array([-2.0, -0.0, 0.0, 3.5])
    np.testing.assert_array_equal(M.moe_activation(h, "relu"), [0.0, 0.0, 0.0, 3.5])
    np.testing.assert_array_equal(M.moe_activation(h, "identity"), h)


def _swiglu_layouts(rng, E=3, I=5, H=7):
    g = (0.4 * rng.standard_normal((E, I, H))).astype(np.float32)
    u = (0.4 * rng.standard_normal((E, I, H))).astype(np.float32)
    gb = (0.1 * rng.standard_normal((E, I))).astype(np.float32)
    ub = (0.1 * rng.standard_normal((E, I))).astype(np.float32)
    inter = np.empty((E, 2 * I, H), np.float32)
    inter[:, 0::2], inter[:, 1::2] = g, u
    inter_b = np.empty((E, 2 * I), np.float32)
    inter_b[:, 0::2], inter_b[:, 1::2] = gb, ub
    concat = np.concatenate([g, u], axis=1)
    concat_b = np.concatenate([gb, ub], axis=1)
    return dict(
        fusion0=dict(fc1_w=g, fc3_w=u, fc1_b=gb, fc3_b=ub),
        fusion1=dict(fc1_w=inter, fc3_w=None, fc1_b=inter_b, fc3_b=None),
        fusion2=dict(fc1_w=concat, fc3_w=None, fc1_b=concat_b, fc3_b=None))


@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (1.702, 1.0)])
def test_swiglu_operand_layouts_agree(alpha, beta):
    # the same gate and linear rows stored separately (FC3), interleaved and
    # concatenated give one result
    rng = np.random.default_rng(1)
    E, I, H, T = 3, 5, 7, 6
    lay = _swiglu_layouts(rng, E, I, H)
    x = rng.standard_normal((T, H)).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    fc2 = (0.4 * rng.standard_normal((E, H, I))).astype(np.float32)
    outs = []
    for f in (0, 1, 2):
        L = lay[f"fusion{f}"]
        outs.append(M.moe(x, logits, L["fc1_w"], fc2, L["fc3_w"], L["fc1_b"], None, L["fc3_b"],
                          attrs=dict(k=2, activation_type="swiglu", swiglu_fusion=f, activation_alpha=alpha,
                                     activation_beta=beta)))
    np.testing.assert_allclose(outs[1], outs[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(outs[2], outs[0], rtol=1e-13, atol=1e-13)


def test_silu_with_fc3_is_swiglu_fusion0_at_defaults():
    rng = np.random.default_rng(2)
    a, _ = _case(rng, act="silu", fc3=True)
    s = M.moe(**a, attrs=dict(k=2, activation_type="silu"))
    g = M.moe(**a, attrs=dict(k=2, activation_type="swiglu", swiglu_fusion=0))
    np.testing.assert_allclose(s, g, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- whole operator
@pytest.mark.parametrize("act", ["relu", "swiglu"])
@pytest.mark.parametrize("normalize", [0, 1])
def test_matches_qmoe_oracle_on_dequantised_weights(act, normalize):
    # QMoE's pinned oracle (MoE routing mode) over dequantised int8 weights
    rng = np.random.default_rng(3)
    T, H, E, I, k = 6, 16, 5, 8, 2
    F = 2 * I if act == "swiglu" else I
    fc1q = rng.integers(0, 256, (E, F, H), dtype=np.uint8)
    fc2q = rng.integers(0, 256, (E, H, I), dtype=np.uint8)
    s1 = rng.uniform(0.01, 0.02, (E, F)).astype(np.float32)
    s2 = rng.uniform(0.01, 0.02, (E, H)).astype(np.float32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    qattrs = dict(k=k, expert_weight_bits=8, activation_type=act, swiglu_fusion=1 if act == "swiglu" else 0,
                  routing="moe", normalize_routing_weights=normalize)
    ref = Q.qmoe(x, logits, fc1q, s1, fc2q, s2, attrs=qattrs)
    w1 = Q.dequantize(fc1q, s1, 8, 0)
    w2 = Q.dequantize(fc2q, s2, 8, 0)
    got = M.moe(x, logits, w1, w2, attrs=dict(k=k, activation_type=act, swiglu_fusion=1 if act == "swiglu" else 0,
                                              normalize_routing_weights=normalize))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_identity_activation_composed_matrices():
    # linear experts: y = W2 (W1 x + b1) + b2 = (W2 W1) x + (W2 b1 + b2)
    rng = np.random.default_rng(4)
    a, attrs = _case(rng, act="identity", k=3, E=5)
    got = M.moe(**a, attrs=attrs)
    sel, w = Q.route(a["logits"], 3, Q.ROUTING_MOE, 0)
    x = a["x"].astype(np.float64)
    ref = np.zeros_like(got)
    for t in range(x.shape[0]):
        for s in range(3):
            e = sel[t, s]
            W = a["fc2_w"][e].astype(np.float64) @ a["fc1_w"][e].astype(np.float64)
            c = a["fc2_w"][e].astype(np.float64) @ a["fc1_b"][e] + a["fc2_b"][e]
            ref[t] += w[t, s] * (W @ x[t] + c)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_fc2_bias_inside_the_weighted_sum():
    rng = np.random.default_rng(5)
    a, attrs = _case(rng, act="gelu", k=2)
    a["fc2_w"] = np.zeros_like(a["fc2_w"])
    got = M.moe(**a, attrs=attrs)
    sel, w = Q.route(a["logits"], 2, Q.ROUTING_MOE, 0)
    ref = (w[:, :, None] * a["fc2_b"][sel].astype(np.float64)).sum(axis=1)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)
    # renormalised weights sum to one: a common bias comes out once
    a["fc2_b"] = np.tile(a["fc2_b"][:1], (a["fc2_b"].shape[0], 1))
    got = M.moe(**a, attrs=dict(attrs, normalize_routing_weights=1))
    np.testing.assert_allclose(got, np.broadcast_to(a["fc2_b"][0], got.shape), rtol=1e-14, atol=1e-15)


def test_zero_inter_gives_weighted_fc2_bias_and_rank3_shape():
    rng = np.random.default_rng(6)
    a, attrs = _case(rng, I=0, act="relu", lead=(2, 3))
    got = M.moe(**a, attrs=attrs)
    assert got.shape == (2, 3, 8)
    sel, w = Q.route(a["logits"], 2, Q.ROUTING_MOE, 0)
    ref = (w[:, :, None] * a["fc2_b"][sel].astype(np.float64)).sum(axis=1)
    np.testing.assert_allclose(got.reshape(6, 8), ref, rtol=1e-14, atol=1e-15)


def test_routed_equals_dense_sum_over_experts():
    # gather form vs every expert on every token masked by the gate matrix
    rng = np.random.default_rng(7)
    a, attrs = _case(rng, T=7, act="swiglu", fusion=2, k=2, E=4)
    got = M.moe(**a, attrs=attrs)
    d = M.moe_validate(**{kk: a[kk] for kk in a}, attrs=attrs)
    sel, w = Q.route(a["logits"], 2, Q.ROUTING_MOE, 0)
    gate = np.zeros((7, 4))
    np.put_along_axis(gate, sel, w, axis=1)
    X = a["x"].astype(np.float64)
    dense = np.zeros_like(got)
    for e in range(4):
        h = X @ a["fc1_w"][e].T.astype(np.float64) + a["fc1_b"][e]
        g, u = h[:, :6], h[:, 6:]
        act = g * sp.expit(g) * u
        y = act @ a["fc2_w"][e].T.astype(np.float64) + a["fc2_b"][e]
        dense += gate[:, e:e + 1] * y
    assert d["F"] == 12
    np.testing.assert_allclose(got, dense, rtol=1e-12, atol=1e-12)


def test_k1_normalised_weight_is_one():
    rng = np.random.default_rng(8)
    a, attrs = _case(rng, k=1)
    _, inter = M.moe(**a, attrs=dict(attrs, k=1, normalize_routing_weights=1), return_intermediates=True)
    np.testing.assert_array_equal(inter["w"], 1.0)
    np.testing.assert_array_equal(inter["sel"][:, 0], np.argmax(a["logits"], axis=1))


# ---------------------------------------------------------------- contract
CONTRACT = [
    ("rank1 input", lambda a: a.update(x=a["x"][0]), {}, "shape"),
    ("logits rows", lambda a: a.update(logits=a["logits"][:-1]), {}, "shape"),
    ("fc2 hidden", lambda a: a.update(fc2_w=a["fc2_w"][:, :-1]), {}, "shape"),
    ("fc1 rows", lambda a: a.update(fc1_w=a["fc1_w"][:, :-1]), {}, "shape"),
    ("fc1 bias", lambda a: a.update(fc1_b=a["fc1_b"][:, :-1]), {}, "shape"),
    ("fc2 bias", lambda a: a.update(fc2_b=a["fc2_b"][:-1]), {}, "shape"),
    ("fc3 shape", lambda a: a.update(fc3_w=np.zeros((4, 6, 7), np.float32)), {}, "shape"),
    ("fc3 bias alone", lambda a: a.update(fc3_b=np.zeros((4, 6), np.float32)), {}, "shape"),
    ("swiglu0 needs fc3", lambda a: None, dict(activation_type="swiglu", swiglu_fusion=0), "shape"),
    ("bad activation", lambda a: None, dict(activation_type="tanh"), "attr"),
    ("bad fusion", lambda a: None, dict(swiglu_fusion=3), "attr"),
    ("k zero", lambda a: None, dict(k=0), "attr"),
    ("k above E", lambda a: None, dict(k=5), "attr"),
    ("normalize 2", lambda a: None, dict(normalize_routing_weights=2), "attr"),
    ("sparse mixer", lambda a: None, dict(use_sparse_mixer=1), "unsupported"),
]


@pytest.mark.parametrize("name,mut,over,kind", CONTRACT, ids=[c[0] for c in CONTRACT])
def test_contract(name, mut, over, kind):
    rng = np.random.default_rng(9)
    a, attrs = _case(rng)
    mut(a)
    with pytest.raises(Q.ContractError) as ei:
        M.moe_validate(**a, attrs=dict(attrs, **over))
    assert ei.value.kind == kind


def test_contract_accepts_unused_fc3_and_fused_shapes():
    rng = np.random.default_rng(10)
    for act, fusion, fc3 in [("relu", 2, True), ("gelu", 0, True), ("swiglu", 1, False), ("swiglu", 2, False),
                             ("swiglu", 0, True), ("silu", 0, False), ("identity", 1, False)]:
        a, attrs = _case(rng, act=act, fusion=fusion, fc3=fc3)
        d = M.moe_validate(**a, attrs=attrs)
        assert d["uses_fc3"] == (fc3 and act in ("silu", "swiglu"))


# ---------------------------------------------------------------- pins have teeth
def _tanh_gelu(h):
    h = np.asarray(h, dtype=np.float64)
    return 0.5 * h * (1 + np.tanh(math.sqrt(2 / math.pi) * (h + 0.044715 * h ** 3)))


def test_planted_mistakes_fail_a_pin(monkeypatch):
    with monkeypatch.context() as m:
        m.setattr(M, "gelu", _tanh_gelu)
        with pytest.raises(AssertionError):
            test_gelu_textbook_values_and_library_cdf()
    real = M.moe_activation

    def swapped(h, act, fusion=0, alpha=1.0, beta=0.0, u3=None, limit=float("inf")):
        if act == "swiglu" and fusion == 2:
            half = h.shape[-1] // 2
            h = np.concatenate([h[..., half:], h[..., :half]], axis=-1)
        return real(h, act, fusion, alpha, beta, u3, limit)
    with monkeypatch.context() as m:
        m.setattr(M, "moe_activation", swapped)
        with pytest.raises(AssertionError):
            test_swiglu_operand_layouts_agree(1.0, 0.0)

    def no_fc2_bias(xrow, e, d, fc1_w, fc2_w, fc3_w=None, fc1_b=None, fc2_b=None, fc3_b=None):
        return real_expert(xrow, e, d, fc1_w, fc2_w, fc3_w, fc1_b, None, fc3_b)
    real_expert = M.moe_expert
    with monkeypatch.context() as m:
        m.setattr(M, "moe_expert", no_fc2_bias)
        with pytest.raises(AssertionError):
            test_identity_activation_composed_matrices()
