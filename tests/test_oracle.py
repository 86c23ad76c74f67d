"""Pins for the CPU oracle, against values the pages and mathematics fix.

Each test ties one part of the oracle to something other than itself: the
GroupedMatMul page's worked examples (hand-derived outputs), a QMoE call that
lifts the page's with_bias example, closed forms for SwiGLU and routing, an
independent brute-force formulation, exact algebraic invariants and a
planted-mistake check that shows each pin actually bites.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import qmoe_oracle as Q
from quantized_mixture_experts_router_amd import workloads as W

from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- P1: GroupedMatMul page examples
@pytest.mark.parametrize("case", _load("grouped_matmul_examples.json")["cases"], ids=lambda c: c["name"])
def test_grouped_matmul_page_examples(case):
    dtypes = case.get("dtypes", ["float32"])
    idx_dtypes = case.get("index_dtypes", ["int64"])
    for dt in dtypes:
        for it in idx_dtypes:
            inp = np.array(case["input"], dtype=dt)
            if "input_shape" in case:
                inp = inp.reshape(case["input_shape"])
            wts = np.array(case["weights"], dtype=dt)
            idx = np.array(case["group_indices"], dtype=it)
            if "group_indices_shape" in case:
                idx = idx.reshape(case["group_indices_shape"])
            elif idx.size == 0:
                idx = idx.reshape(inp.shape[0], 0)
            bias = None if case["bias"] is None else np.array(case["bias"], dtype=dt)
            out = oracle.grouped_matmul(inp, wts, idx, bias)
            assert out.shape == tuple(case["expected_shape"])
            assert out.dtype == np.dtype(dt)
            if case["expected"] is not None:
                tol = 1e-3 if dt == "float16" else 1e-6
                np.testing.assert_allclose(out.astype(np.float64), np.array(case["expected"]), atol=tol, rtol=0)


def test_grouped_matmul_rejects_bad_index():
    with pytest.raises(ValueError):
        oracle.grouped_matmul(np.ones((1, 2)), np.ones((2, 2, 2)), np.array([[2]]))
    with pytest.raises(ValueError):
        oracle.grouped_matmul(np.ones((1, 2)), np.ones((2, 2, 2)), np.array([[-1]]))


@pytest.mark.parametrize("case", _load("grouped_matmul_examples.json")["cases"], ids=lambda c: c["name"])
def test_grouped_matmul_rows_page_examples(case):
    # the row-sampled form reproduces the page's examples too
    if case["expected"] is None:
        return
    inp = np.array(case["input"], dtype=np.float64)
    if "input_shape" in case:
        inp = inp.reshape(case["input_shape"])
    wts = np.array(case["weights"], dtype=np.float64)
    idx = np.array(case["group_indices"], dtype=np.int64)
    if "group_indices_shape" in case:
        idx = idx.reshape(case["group_indices_shape"])
    elif idx.size == 0:
        idx = idx.reshape(inp.shape[0], 0)
    bias = None if case["bias"] is None else np.array(case["bias"], dtype=np.float64)
    out = oracle.grouped_matmul_rows(inp, wts, idx, bias)
    np.testing.assert_allclose(out, np.array(case["expected"]).reshape(out.shape), atol=1e-12, rtol=0)


@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_matmul_rows_agrees_with_loops(seed):
    rng = np.random.default_rng(seed)
    M, K, G, N, S = 5, 7, 3, 4, 2
    inp = rng.standard_normal((M, K)).astype(np.float32)
    wts = rng.standard_normal((G, K, N)).astype(np.float32)
    bias = rng.standard_normal((G, N)).astype(np.float32)
    idx = rng.integers(0, G, size=(M, S))
    full = oracle.grouped_matmul(inp, wts, idx, bias, out_dtype=np.float64)
    np.testing.assert_allclose(oracle.grouped_matmul_rows(inp, wts, idx, bias), full, rtol=1e-13, atol=1e-13)
    rows = np.array([4, 1])
    np.testing.assert_allclose(oracle.grouped_matmul_rows(inp, wts, idx, None, rows),
                               oracle.grouped_matmul(inp, wts, idx, None, out_dtype=np.float64)[rows],
                               rtol=1e-13, atol=1e-13)


def test_grouped_matmul_closed_forms():
    # identity weights give the input back; a one-hot column picks one input
    # element; bias alone (K == 0) is the result
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 4))
    eye = np.stack([np.eye(4), 2 * np.eye(4)])
    idx = np.array([[0, 1], [1, 1], [0, 0]])
    for f in (oracle.grouped_matmul, oracle.grouped_matmul_rows):
        out = f(x, eye, idx)
        np.testing.assert_array_equal(out[:, 0], x * np.array([1, 2, 1])[:, None])
        np.testing.assert_array_equal(out[:, 1], x * np.array([2, 2, 1])[:, None])
        b = rng.standard_normal((2, 5))
        out0 = f(np.zeros((3, 0)), np.zeros((2, 0, 5)), idx, b)
        np.testing.assert_array_equal(out0, b[idx])
    with pytest.raises(ValueError):
        oracle.grouped_matmul_rows(np.ones((1, 2)), np.ones((2, 2, 2)), np.array([[-1]]))


# ---------------------------------------------------------------- P2: lifted with_bias example
def _lifted_arrays():
    g = _load("qmoe_lifted_with_bias.json")
    x = np.array(g["input"], dtype=np.float32)
    logits = np.array(g["router_probs"], dtype=np.float32)
    fc1 = np.array(g["fc1_codes"], dtype=np.uint8)
    fc2 = np.array(g["fc2_codes"], dtype=np.uint8)
    fc1_s = np.full(fc1.shape[:2], g["fc1_scale"], dtype=np.float32)
    fc2_s = np.full(fc2.shape[:2], g["fc2_scale"], dtype=np.float32)
    return g, (x, logits, fc1, fc1_s, fc2, fc2_s)


def test_lifted_with_bias_example():
    g, arrs = _lifted_arrays()
    out, inter = oracle.qmoe(*arrs, attrs=g["attrs"], return_intermediates=True)
    np.testing.assert_array_equal(inter["sel"], np.array(g["expected_selection"]))
    np.testing.assert_allclose(inter["w"], np.array(g["expected_weights"]), atol=1e-15)
    np.testing.assert_allclose(out, np.array(g["expected_output"]), atol=g["tolerance"], rtol=0)
    dense = oracle.qmoe_dense(*arrs, attrs=g["attrs"])
    np.testing.assert_allclose(dense, np.array(g["expected_output"]), atol=g["tolerance"], rtol=0)


def test_relu_negative_branch_example():
    # ReLU's negative branch: one FC1 output of every selected expert is
    # negative and must be zeroed (hand-worked values in the fixture)
    g = _load("qmoe_relu_negative.json")
    x = np.array(g["input"], dtype=np.float32)
    logits = np.array(g["router_probs"], dtype=np.float32)
    fc1 = np.array(g["fc1_codes"], dtype=np.uint8)
    fc2 = np.array(g["fc2_codes"], dtype=np.uint8)
    arrs = (x, logits, fc1, np.full(fc1.shape[:2], g["fc1_scale"], dtype=np.float32), fc2,
            np.full(fc2.shape[:2], g["fc2_scale"], dtype=np.float32))
    out, inter = oracle.qmoe(*arrs, attrs=g["attrs"], return_intermediates=True)
    np.testing.assert_array_equal(inter["sel"], np.array(g["expected_selection"]))
    np.testing.assert_allclose(out, np.array(g["expected_output"]), atol=g["tolerance"], rtol=0)
    dense = oracle.qmoe_dense(*arrs, attrs=g["attrs"])
    np.testing.assert_allclose(dense, np.array(g["expected_output"]), atol=g["tolerance"], rtol=0)


# ---------------------------------------------------------------- SwiGLU closed forms
@pytest.mark.parametrize("ci", [0, 1])
def test_swiglu_interleave_closed_form(ci):
    g = _load("swiglu_interleave.json")
    c = g["cases"][ci]
    x = np.array(g["input"], dtype=np.float32)
    logits = np.array(g["router_probs"], dtype=np.float32)
    fc1 = np.array(g["fc1_codes"], dtype=np.uint8)
    fc2 = np.array(g["fc2_codes"], dtype=np.uint8)
    fc1_s = np.full(fc1.shape[:2], g["fc1_scale"], dtype=np.float32)
    fc2_s = np.full(fc2.shape[:2], g["fc2_scale"], dtype=np.float32)
    attrs = dict(k=1, expert_weight_bits=8, activation_type="swiglu", swiglu_fusion=1,
                 activation_alpha=c["alpha"], activation_beta=c["beta"])
    out = oracle.qmoe(x, logits, fc1, fc1_s, fc2, fc2_s, attrs)
    assert abs(out[0, 0] - c["expected_out0"]) < g["tolerance"]
    assert out[0, 1] == 0.0
    if "swapped_reading" in c:
        assert abs(out[0, 0] - c["swapped_reading"]) > 0.1


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("case", _load("route_ties.json")["cases"])
def test_route_ties_and_order(case):
    L = np.array(case["logits"], dtype=np.float32)
    sel, w = oracle.route(L, case["k"])
    np.testing.assert_array_equal(sel, np.array(case["expected"]))
    np.testing.assert_allclose(w, np.array(case["weights"]), rtol=1e-7, atol=0)


def test_route_k1_weight_is_exactly_one():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((200, 7)).astype(np.float32)
    sel, w = oracle.route(L, 1)
    assert np.all(w == 1.0)
    np.testing.assert_array_equal(sel[:, 0], np.argmax(L, axis=1))


def test_route_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((50, 6)).astype(np.float32) * 3
    sel, w = oracle.route(L, 6, "qmoe")
    L64 = L.astype(np.float64)
    for t in range(L.shape[0]):
        full = [math.exp(v) for v in L64[t]]
        s = sum(full)
        for j in range(6):
            assert abs(w[t, j] - full[sel[t, j]] / s) < 1e-14
    sel2, w2 = oracle.route(L, 6, "moe", normalize=0)
    np.testing.assert_array_equal(sel, sel2)
    np.testing.assert_allclose(w, w2, atol=1e-14)


def test_moe_normalized_equals_qmoe_weights():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((80, 9)).astype(np.float32) * 2
    for k in (1, 2, 4, 9):
        s1, w1 = oracle.route(L, k, "qmoe")
        s2, w2 = oracle.route(L, k, "moe", normalize=1)
        np.testing.assert_array_equal(s1, s2)
        np.testing.assert_allclose(w1, w2, atol=1e-12)
        _, w3 = oracle.route(L, k, "moe", normalize=0)
        assert np.all(w3.sum(axis=1) <= 1 + 1e-12)


def test_route_sum_to_one_and_descending():
    rng = np.random.default_rng(6)
    L = rng.standard_normal((300, 16)).astype(np.float32)
    sel, w = oracle.route(L, 5)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)
    vals = np.take_along_axis(L, sel, axis=1)
    assert np.all(np.diff(vals, axis=1) <= 0)
    # brute force: the selected set is the k largest
    for t in range(L.shape[0]):
        thr = np.sort(L[t])[::-1][4]
        assert set(sel[t]) == set(np.nonzero(L[t] >= thr)[0][:5]) or np.all(L[t][sel[t]] >= thr)


# ---------------------------------------------------------------- dequantisation and packing
def test_nibble_order_convention():
    g = _load("nibble_order.json")
    b = np.array(g["bytes"], dtype=np.uint8)
    np.testing.assert_array_equal(Q.unpack_codes(b, 4), g["codes_4bit"])
    np.testing.assert_array_equal(Q.dequantize(b[None], np.ones(1), 4, 0)[0], g["dequant_4bit_scale1"])
    np.testing.assert_array_equal(Q.unpack_codes(b, 8), g["codes_8bit"])
    np.testing.assert_array_equal(Q.dequantize(b[None], np.ones(1), 8, 0)[0], g["dequant_8bit_scale1"])


def test_blockwise_scale_indexing():
    # 8-bit codes all 129 (value +1) over K = 64 with block 16: W[n, c] = scale[n, c // 16]
    packed = np.full((2, 64), 129, dtype=np.uint8)
    s = np.array([[1, 2, 3, 4], [5, 6, 7, 8]], dtype=np.float32)
    Wd = Q.dequantize(packed, s, 8, 16)
    for n in range(2):
        for c in range(64):
            assert Wd[n, c] == s[n, c // 16]


def _tiny(rng, bits, bs, act, k, rank3, E=4, H=32, I=32, T=6):
    shape = (2, T // 2) if rank3 else (T,)
    return W.random_case(rng, tokens_shape=shape, hidden=H, experts=E, inter=I, k=k, bits=bits,
                         block_size=bs, activation=act)


# ---------------------------------------------------------------- P3 / P5: routed == dense brute force
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("bs", [0, 16, 32])
@pytest.mark.parametrize("act", ["relu", "swiglu"])
def test_routed_equals_dense_bruteforce(bits, bs, act):
    rng = np.random.default_rng(100 + bits + bs + (act == "swiglu"))
    for k in (1, 2, 4):
        for rank3 in (False, True):
            w, a = _tiny(rng, bits, bs, act, k, rank3)
            attrs = w.attrs()
            out = oracle.qmoe(*a.values(), attrs=attrs)
            dense = oracle.qmoe_dense(*a.values(), attrs=attrs)
            assert out.shape == a["input"].shape
            np.testing.assert_allclose(out, dense, rtol=1e-10, atol=1e-12)
            sub = oracle.qmoe_tokens([0, 3, 5], *a.values(), attrs=attrs)
            np.testing.assert_allclose(sub, out.reshape(-1, w.hidden)[[0, 3, 5]], rtol=1e-10, atol=1e-12)


def test_k1_equals_argmax_expert_ffn():
    rng = np.random.default_rng(11)
    w, a = _tiny(rng, 8, 0, "relu", 1, False, E=5)
    out = oracle.qmoe(*a.values(), attrs=w.attrs())
    for t in range(w.tokens):
        e = int(np.argmax(a["router_probs"][t]))
        W1 = Q.dequantize(a["fc1_experts_weights"][e], a["fc1_scales"][e], 8, 0)
        W2 = Q.dequantize(a["fc2_experts_weights"][e], a["fc2_scales"][e], 8, 0)
        # the expert FFN written per element
        xt = a["input"][t].astype(np.float64)
        h = [max(sum(W1[j, c] * xt[c] for c in range(w.hidden)), 0.0) for j in range(w.inter)]
        y = [sum(W2[c, j] * h[j] for j in range(w.inter)) for c in range(w.hidden)]
        np.testing.assert_allclose(out[t], y, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- P7: exact invariants
def test_all_midpoint_codes_give_zero():
    rng = np.random.default_rng(12)
    for bits in (4, 8):
        w, a = _tiny(rng, bits, 16, "swiglu", 2, False)
        a["fc1_experts_weights"][:] = 0x88 if bits == 4 else 128
        out = oracle.qmoe(*a.values(), attrs=w.attrs())
        assert np.all(out == 0.0)


def test_scale_doubling_is_exact():
    rng = np.random.default_rng(13)
    w, a = _tiny(rng, 4, 16, "relu", 2, False)
    base = oracle.qmoe(*a.values(), attrs=w.attrs())
    b = dict(a)
    b["fc2_scales"] = a["fc2_scales"] * 2
    np.testing.assert_array_equal(oracle.qmoe(*b.values(), attrs=w.attrs()), 2 * base)
    c = dict(a)
    c["fc1_scales"] = a["fc1_scales"] * 2
    np.testing.assert_array_equal(oracle.qmoe(*c.values(), attrs=w.attrs()), 2 * base)


def test_4bit_reencoded_as_8bit_is_identical():
    rng = np.random.default_rng(14)
    w, a = _tiny(rng, 4, 0, "swiglu", 2, False)
    q1 = Q.unpack_codes(a["fc1_experts_weights"], 4)
    q2 = Q.unpack_codes(a["fc2_experts_weights"], 4)
    b = dict(a)
    b["fc1_experts_weights"] = (q1 + 120).astype(np.uint8)
    b["fc2_experts_weights"] = (q2 + 120).astype(np.uint8)
    attrs8 = dict(w.attrs(), expert_weight_bits=8)
    np.testing.assert_array_equal(oracle.qmoe(*a.values(), attrs=w.attrs()), oracle.qmoe(*b.values(), attrs=attrs8))


def test_equal_block_scales_match_columnwise():
    rng = np.random.default_rng(15)
    w, a = _tiny(rng, 4, 0, "swiglu", 2, False)
    b = dict(a)
    b["fc1_scales"] = np.repeat(a["fc1_scales"][..., None], w.hidden // 16, axis=-1)
    b["fc2_scales"] = np.repeat(a["fc2_scales"][..., None], w.inter // 16, axis=-1)
    attrs = dict(w.attrs(), block_size=16)
    np.testing.assert_array_equal(oracle.qmoe(*a.values(), attrs=w.attrs()), oracle.qmoe(*b.values(), attrs=attrs))


# ---------------------------------------------------------------- P8: permutation structure
def test_permutation_structure_and_stability():
    rng = np.random.default_rng(16)
    for E, T, k in ((4, 10, 2), (16, 257, 3), (64, 1000, 6)):
        L = rng.standard_normal((T, E)).astype(np.float32)
        sel, _ = oracle.route(L, k)
        counts, offsets, perm = oracle.expert_permutation(sel, E)
        assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
        assert np.all(np.diff(offsets) == counts)
        assert sorted(perm.tolist()) == list(range(T * k))
        flat = sel.reshape(-1)
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(flat[seg] == e)
            assert np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------- P9: symmetries
def test_token_permutation_and_expert_relabeling():
    rng = np.random.default_rng(17)
    w, a = _tiny(rng, 4, 16, "swiglu", 2, False, E=5, T=8)
    base = oracle.qmoe(*a.values(), attrs=w.attrs())
    pt = rng.permutation(w.tokens)
    b = dict(a, input=a["input"][pt], router_probs=a["router_probs"][pt])
    np.testing.assert_allclose(oracle.qmoe(*b.values(), attrs=w.attrs()), base[pt], rtol=1e-12, atol=1e-14)
    pe = rng.permutation(w.experts)
    c = dict(a, router_probs=a["router_probs"][:, pe], fc1_experts_weights=a["fc1_experts_weights"][pe],
             fc1_scales=a["fc1_scales"][pe], fc2_experts_weights=a["fc2_experts_weights"][pe],
             fc2_scales=a["fc2_scales"][pe])
    np.testing.assert_allclose(oracle.qmoe(*c.values(), attrs=w.attrs()), base, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- edge cases
def test_zero_inter_gives_zeros_and_zero_tokens_gives_empty():
    rng = np.random.default_rng(18)
    w, a = _tiny(rng, 8, 0, "relu", 1, False, I=0)
    out = oracle.qmoe(*a.values(), attrs=w.attrs())
    assert out.shape == a["input"].shape and np.all(out == 0)
    w2, b = _tiny(rng, 8, 0, "relu", 1, False)
    b["input"] = b["input"][:0]
    b["router_probs"] = b["router_probs"][:0]
    out2 = oracle.qmoe(*b.values(), attrs=w2.attrs())
    assert out2.shape == (0, w2.hidden)


CONTRACT_CASES = [
    ("k0", dict(k=0), None, "attr"),
    ("k_gt_e", dict(k=5), None, "attr"),
    ("bits2", dict(expert_weight_bits=2), None, "attr"),
    ("normalize2", dict(normalize_routing_weights=2), None, "attr"),
    ("prepacked1", dict(weights_prepacked=1), None, "unsupported"),
    ("prepacked2", dict(weights_prepacked=2), None, "attr"),
    ("sparse", dict(use_sparse_mixer=1), None, "unsupported"),
    ("quant_fp", dict(quant_type="fp"), None, "unsupported"),
    ("relu_fused", dict(swiglu_fusion=1), None, "attr"),
    ("fusion2", dict(swiglu_fusion=2), None, "unsupported"),
    ("bs8", dict(block_size=8), None, "attr"),
    ("bs24", dict(block_size=24), None, "attr"),
    ("bs64_not_dividing", dict(block_size=64), "blocks64", "shape"),
    ("router_rows", {}, "router_rows", "shape"),
    ("fc2_rows", {}, "fc2_rows", "shape"),
    ("packed_cols", {}, "packed_cols", "shape"),
    ("scale_rank", {}, "scale_rank", "shape"),
    ("dtype", {}, "dtype", "dtype"),
    ("rank4", {}, "rank4", "shape"),
]


@pytest.mark.parametrize("name,attr_over,mut,kind", CONTRACT_CASES, ids=[c[0] for c in CONTRACT_CASES])
def test_contract_violations(name, attr_over, mut, kind):
    rng = np.random.default_rng(19)
    w, a = _tiny(rng, 4, 0, "relu", 1, False)
    attrs = dict(w.attrs(), **attr_over)
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
    with pytest.raises(Q.ContractError) as ei:
        oracle.validate(*a.values(), attrs=attrs)
    assert ei.value.kind == kind


# ---------------------------------------------------------------- planted mistakes must fail a pin
def _swap_nibbles(packed, bits):
    b = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return b.astype(np.int64)
    q = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int64)
    q[..., 0::2] = b >> 4
    q[..., 1::2] = b & 0x0F
    return q


def _gate_odd(h, act, alpha=1.0, beta=0.0):
    h = np.asarray(h, dtype=np.float64)
    if act == "relu":
        return np.maximum(h, 0)
    g, u = h[..., 1::2], h[..., 0::2]
    return g / (1 + np.exp(-alpha * g)) * (u + beta)


def _ffn_transposed(xrows, w1, w2, act, alpha, beta):
    # FC1 read as x @ W1 for square shapes (the GroupedMatMul [K, N] orientation)
    h = np.asarray(xrows, dtype=np.float64) @ w1
    return Q.activation(h, act, alpha, beta) @ w2.T


def _full_softmax_route(orig_route):
    def route(logits, k, routing="qmoe", normalize=0):
        sel, _ = orig_route(logits, k, routing, normalize)
        L = np.asarray(logits, dtype=np.float64)
        p = np.exp(L - L.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        return sel, np.take_along_axis(p, sel, axis=1)
    return route


def _pins_pass():
    """Run the value pins; return False if any of them fails."""
    try:
        test_lifted_with_bias_example()
        test_relu_negative_branch_example()
        test_swiglu_interleave_closed_form(0)
        test_nibble_order_convention()
        for c in _load("route_ties.json")["cases"]:
            test_route_ties_and_order(c)
    except Exception:  # an assertion, or a shape error from a transposed operand
        return False
    return True


def _relu_leaky(h, act, alpha=1.0, beta=0.0, limit=float("inf")):
    # ReLU without its clamp (identity on negative values)
    if act == "relu":
        return np.asarray(h, dtype=np.float64)
    return _orig_activation(h, act, alpha, beta, limit)


_orig_activation = Q.activation


@pytest.mark.parametrize("mutation", ["nibbles", "gate_odd", "fc1_transposed", "full_softmax", "no_midpoint",
                                      "relu_no_clamp"])
def test_planted_mistakes_fail_a_pin(monkeypatch, mutation):
    assert _pins_pass()
    if mutation == "nibbles":
        monkeypatch.setattr(Q, "unpack_codes", _swap_nibbles)
    elif mutation == "gate_odd":
        monkeypatch.setattr(Q, "activation", _gate_odd)
    elif mutation == "fc1_transposed":
        monkeypatch.setattr(Q, "expert_ffn", _ffn_transposed)
        monkeypatch.setattr(oracle, "qmoe", Q.qmoe)
    elif mutation == "full_softmax":
        wrong = _full_softmax_route(Q.route)
        monkeypatch.setattr(Q, "route", wrong)
        monkeypatch.setattr(oracle, "route", wrong)
    elif mutation == "relu_no_clamp":
        monkeypatch.setattr(Q, "activation", _relu_leaky)
    elif mutation == "no_midpoint":
        def no_mid(packed, scales, bits, bs):
            q = Q.unpack_codes(packed, bits).astype(np.float64)
            s = np.asarray(scales, dtype=np.float64)
            return q * (s[..., None] if bs == 0 else np.repeat(s, bs, axis=-1))
        monkeypatch.setattr(Q, "dequantize", no_mid)
    assert not _pins_pass()
