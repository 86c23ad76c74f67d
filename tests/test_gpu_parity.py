"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact routing indices, counts, offsets and permutation; routing weights
within 1e-6; outputs within 2e-3 x RMS of the oracle's output.  Small cases
compare every element; the full-size workloads compare the routing exactly
and a sample of output rows that the oracle computes one by one.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import qmoe_oracle as Q
from quantized_mixture_experts_router_amd import workloads as W

from conftest import GOLDEN
from gpu_util import OUT_TOL, check_output, check_routing, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _full_check(w, a, torch, label):
    attrs = w.attrs()
    say(f"[case] {label} T={w.tokens} H={w.hidden} E={w.experts} I={w.inter} k={w.k} bits={w.bits} "
        f"bs={w.block_size} act={w.activation}")
    res = run_gpu(a, attrs, torch)
    ref, inter = oracle.qmoe(*a.values(), attrs=attrs, return_intermediates=True)
    check_routing(res, inter["sel"], inter["w"], inter["counts"], inter["offsets"], inter["perm"])
    return check_output(res["out"], ref, label)


def test_tiny_workload_every_element(torch):
    w = W.WORKLOADS["tiny"]
    _full_check(w, W.generate(w), torch, "tiny")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_lifted_with_bias_example(torch):
    g = _golden("qmoe_lifted_with_bias.json")
    fc1 = np.array(g["fc1_codes"], dtype=np.uint8)
    fc2 = np.array(g["fc2_codes"], dtype=np.uint8)
    a = dict(input=np.array(g["input"], dtype=np.float32),
             router_probs=np.array(g["router_probs"], dtype=np.float32),
             fc1_experts_weights=fc1, fc1_scales=np.full(fc1.shape[:2], g["fc1_scale"], dtype=np.float32),
             fc2_experts_weights=fc2, fc2_scales=np.full(fc2.shape[:2], g["fc2_scale"], dtype=np.float32))
    res = run_gpu(a, dict(g["attrs"]), torch)
    np.testing.assert_array_equal(res["topk_idx"].reshape(2, 2), np.array(g["expected_selection"]))
    np.testing.assert_allclose(res["topk_w"].reshape(2, 2), g["expected_weights"], atol=1e-7)
    np.testing.assert_allclose(res["out"], np.array(g["expected_output"]), atol=g["tolerance"], rtol=0)


def test_relu_negative_branch_example(torch):
    g = _golden("qmoe_relu_negative.json")
    fc1 = np.array(g["fc1_codes"], dtype=np.uint8)
    fc2 = np.array(g["fc2_codes"], dtype=np.uint8)
    a = dict(input=np.array(g["input"], dtype=np.float32),
             router_probs=np.array(g["router_probs"], dtype=np.float32),
             fc1_experts_weights=fc1, fc1_scales=np.full(fc1.shape[:2], g["fc1_scale"], dtype=np.float32),
             fc2_experts_weights=fc2, fc2_scales=np.full(fc2.shape[:2], g["fc2_scale"], dtype=np.float32))
    res = run_gpu(a, dict(g["attrs"]), torch)
    np.testing.assert_array_equal(res["topk_idx"].reshape(2, 2), np.array(g["expected_selection"]))
    np.testing.assert_allclose(res["out"], np.array(g["expected_output"]), atol=g["tolerance"], rtol=0)


def test_swiglu_closed_form(torch):
    g = _golden("swiglu_interleave.json")
    fc1 = np.array(g["fc1_codes"], dtype=np.uint8)
    fc2 = np.array(g["fc2_codes"], dtype=np.uint8)
    a = dict(input=np.array(g["input"], dtype=np.float32),
             router_probs=np.array(g["router_probs"], dtype=np.float32),
             fc1_experts_weights=fc1, fc1_scales=np.full(fc1.shape[:2], g["fc1_scale"], dtype=np.float32),
             fc2_experts_weights=fc2, fc2_scales=np.full(fc2.shape[:2], g["fc2_scale"], dtype=np.float32))
    for c in g["cases"]:
        attrs = dict(k=1, expert_weight_bits=8, activation_type="swiglu", swiglu_fusion=1,
                     activation_alpha=c["alpha"], activation_beta=c["beta"])
        res = run_gpu(a, attrs, torch)
        assert abs(float(res["out"][0, 0]) - c["expected_out0"]) <= 2e-6 * abs(c["expected_out0"])
        assert res["out"][0, 1] == 0.0


def test_route_ties_through_gpu(torch):
    g = _golden("route_ties.json")
    for c in g["cases"]:
        L = np.array(c["logits"], dtype=np.float32)
        E = L.shape[1]
        rng = np.random.default_rng(1)
        w = W.Workload("ties", (1, 32), E, 32, c["k"], 8, 0, "relu", (0.01, 0.02))
        a = W.generate(w, seed=3)
        a["router_probs"] = L
        res = run_gpu(a, w.attrs(), torch)
        np.testing.assert_array_equal(res["topk_idx"].reshape(1, -1), np.array(c["expected"]))
        np.testing.assert_allclose(res["topk_w"].reshape(1, -1), np.array(c["weights"]), rtol=2e-6, atol=0)
        del rng


# Small sweeps: every element.  (T, H, E, I, k) chosen to cover one and several
# M tiles on the weight-streaming path (up to 224 tokens where its stages
# tile both reductions), the LDS-tiled path (larger T,
# H and I multiples of 64) and the register-tiled path (other shapes), ragged
# tails in every dimension, unused experts and k = E.
SHAPES = [
    (1, 64, 4, 32, 1), (5, 128, 3, 64, 2), (16, 256, 8, 96, 2), (17, 64, 4, 160, 3),
    (33, 128, 6, 64, 6), (64, 192, 8, 128, 2), (70, 128, 5, 96, 2), (200, 64, 16, 64, 4),
    (300, 256, 1, 32, 1), (24, 512, 8, 256, 3), (40, 256, 4, 256, 2), (60, 256, 4, 128, 2),
    (130, 128, 3, 192, 2), (257, 320, 4, 128, 3),
    # either side of the streaming / tiled switches: 224 tokens where both
    # GEMMs stream (16-row streaming tiles, experts spread over many tiles),
    # 64 where only FC1 does (int4: FC2's 256-code reduction is not a whole
    # 512-code stage), then 128-row LDS tiles
    (224, 512, 4, 512, 2), (225, 512, 4, 512, 2), (64, 512, 8, 256, 2), (65, 512, 8, 256, 2),
]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("bs", [0, 16, 32, 64])
@pytest.mark.parametrize("act", ["relu", "swiglu"])
def test_small_sweep(torch, bits, bs, act):
    rng = np.random.default_rng(1000 + bits * 10 + bs + (act == "swiglu"))
    for (T, H, E, I, k) in SHAPES:
        if bs and (H % bs or I % bs):
            continue
        shape = (T,) if T % 2 else (2, T // 2)
        w, a = W.random_case(rng, tokens_shape=shape, hidden=H, experts=E, inter=I, k=k, bits=bits,
                             block_size=bs, activation=act)
        _full_check(w, a, torch, f"sweep T{T} H{H} E{E} I{I} k{k}")


# Weight streaming in tiles of 8 rows (single stages of 8 items: 2048 codes
# at 4 bits, 1024 at 8), taken when routing gives an expert at most 4 rows on
# average: (T, H, E, I, k, bits, bs, act, logit bias of expert 0, forced tile
# rows).  A bias makes expert 0 draw most tokens, so it spans several tiles;
# forcing 8-row tiles at larger batches gives every expert several.
EIGHT_ROW = [
    (16, 2048, 8, 2048, 2, 4, 64, "swiglu", 0.0, None),
    (16, 2048, 8, 2048, 2, 4, 64, "swiglu", 4.0, None),
    (13, 2048, 8, 4096, 2, 4, 128, "relu", 0.0, None),
    (16, 2048, 8, 2048, 2, 4, 0, "swiglu", 2.0, None),
    (12, 1024, 8, 2048, 2, 8, 0, "swiglu", 0.0, None),
    (12, 1024, 8, 1024, 2, 8, 32, "relu", 3.0, None),
    (10, 2048, 6, 2048, 2, 8, 64, "swiglu", 0.0, None),
    (1, 2048, 4, 2048, 1, 4, 64, "swiglu", 0.0, None),
    (40, 2048, 4, 2048, 2, 4, 64, "swiglu", 0.0, "8"),
    (30, 1024, 3, 1024, 3, 8, 32, "relu", 0.0, "8"),
]


@pytest.mark.parametrize("items", ["1", "4", "8"])
@pytest.mark.parametrize("case", EIGHT_ROW)
def test_stream_eight_row_tiles(torch, monkeypatch, case, items):
    """Every stage length of 8-row tiles (QMOE_STREAM_STAGE_ITEMS; the plan
    itself takes the longest stage that still fills the chip)."""
    import quantized_mixture_experts_router_amd as qm
    T, H, E, I, k, bits, bs, act, bias, force = case
    if force:
        monkeypatch.setenv("QMOE_STREAM_TILE_ROWS", force)
    monkeypatch.setenv("QMOE_STREAM_STAGE_ITEMS", items)
    rng = np.random.default_rng(1300 + T + E + bits + bs)
    w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, bits=bits, block_size=bs,
                         activation=act)
    a["router_probs"] = a["router_probs"].copy()
    a["router_probs"][:, 0] += bias
    plan = qm.qmoe_plan_describe(*a.values(), attrs=w.attrs())
    assert "fc1=stream fc2=stream" in plan and "tile_rows=8 " in plan and f"s1=1:{items}:" in plan, plan
    _full_check(w, a, torch, f"8-row tiles T{T} H{H} E{E} I{I} k{k} bits{bits} bs{bs} {act} bias{bias} ({plan})")


def test_front_end_paths(torch):
    """Routing and permutation on both front ends: one workgroup (up to 1024
    slots and 1024 experts) and the chunked multi-kernel path beyond."""
    rng = np.random.default_rng(76)
    for (T, E, k) in [(512, 8, 2), (205, 16, 5), (4, 1024, 3), (300, 1000, 3), (64, 300, 16), (700, 1024, 2)]:
        w, a = W.random_case(rng, tokens_shape=(T,), hidden=64, experts=E, inter=16, k=k, bits=8,
                             block_size=0, activation="relu")
        _full_check(w, a, torch, f"front end T{T} E{E} k{k} (slots {T * k})")


def test_unaligned_shapes(torch):
    rng = np.random.default_rng(77)
    # H or I not a multiple of 8 takes the byte-load path
    for (T, H, E, I, k, bits) in [(3, 6, 2, 4, 1, 4), (9, 20, 3, 12, 2, 8), (70, 36, 4, 10, 2, 4), (5, 3, 2, 5, 2, 8)]:
        for act in ("relu", "swiglu"):
            w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, bits=bits,
                                 block_size=0, activation=act)
            _full_check(w, a, torch, f"unaligned T{T} H{H} I{I} bits{bits} {act}")


def test_moe_routing_modes(torch):
    rng = np.random.default_rng(78)
    for normalize in (0, 1):
        for k in (1, 3, 8):
            w, a = W.random_case(rng, tokens_shape=(40,), hidden=64, experts=8, inter=64, k=k, bits=4,
                                 block_size=32, activation="swiglu", logit_sigma=2.0)
            attrs = dict(w.attrs(), routing="moe", normalize_routing_weights=normalize)
            res = run_gpu(a, attrs, torch)
            ref, inter = oracle.qmoe(*a.values(), attrs=attrs, return_intermediates=True)
            check_routing(res, inter["sel"], inter["w"], inter["counts"], inter["offsets"], inter["perm"],
                          selected_softmax=bool(normalize))
            check_output(res["out"], ref, f"moe normalize={normalize} k={k}")


def test_alpha_beta(torch):
    rng = np.random.default_rng(79)
    w, a = W.random_case(rng, tokens_shape=(24,), hidden=128, experts=4, inter=64, k=2, bits=8,
                         block_size=0, activation="swiglu")
    attrs = dict(w.attrs(), activation_alpha=1.702, activation_beta=1.0)
    res = run_gpu(a, attrs, torch)
    check_output(res["out"], oracle.qmoe(*a.values(), attrs=attrs), "alpha=1.702 beta=1")


# ------------------------------------------------------------------ exact invariants on the GPU
def test_all_midpoint_codes_give_exact_zero(torch):
    rng = np.random.default_rng(80)
    for bits in (4, 8):
        w, a = W.random_case(rng, tokens_shape=(20,), hidden=64, experts=4, inter=64, k=2, bits=bits,
                             block_size=32, activation="swiglu")
        a["fc1_experts_weights"][:] = 0x88 if bits == 4 else 128
        res = run_gpu(a, w.attrs(), torch)
        assert np.all(res["out"] == 0.0)


def test_scale_doubling_doubles_output_bitwise(torch):
    rng = np.random.default_rng(81)
    for bs in (0, 32):
        w, a = W.random_case(rng, tokens_shape=(40,), hidden=128, experts=4, inter=64, k=2, bits=4,
                             block_size=bs, activation="relu")
        r1 = run_gpu(a, w.attrs(), torch)["out"]
        b = dict(a, fc2_scales=a["fc2_scales"] * 2)
        r2 = run_gpu(b, w.attrs(), torch)["out"]
        np.testing.assert_array_equal(r2, 2 * r1)


def test_4bit_reencoded_as_8bit(torch):
    rng = np.random.default_rng(82)
    w, a = W.random_case(rng, tokens_shape=(30,), hidden=128, experts=4, inter=64, k=2, bits=4,
                         block_size=0, activation="swiglu")
    q1 = Q.unpack_codes(a["fc1_experts_weights"], 4)
    q2 = Q.unpack_codes(a["fc2_experts_weights"], 4)
    b = dict(a, fc1_experts_weights=(q1 + 120).astype(np.uint8), fc2_experts_weights=(q2 + 120).astype(np.uint8))
    r4 = run_gpu(a, w.attrs(), torch)["out"]
    r8 = run_gpu(b, dict(w.attrs(), expert_weight_bits=8), torch)["out"]
    ref = oracle.qmoe(*a.values(), attrs=w.attrs())
    check_output(r4, ref, "4-bit")
    check_output(r8, ref, "same codes as 8-bit")


def test_determinism_bitwise(torch):
    w = W.WORKLOADS["tiny"]
    a = W.generate(w)
    r1 = run_gpu(a, w.attrs(), torch)
    r2 = run_gpu(a, w.attrs(), torch)
    for key in r1:
        np.testing.assert_array_equal(r1[key], r2[key])


# ------------------------------------------------------------------ edge cases and errors
def test_zero_tokens_and_zero_inter(torch):
    rng = np.random.default_rng(83)
    w, a = W.random_case(rng, tokens_shape=(6,), hidden=64, experts=4, inter=0, k=2, bits=8, block_size=0,
                         activation="relu")
    res = run_gpu(a, w.attrs(), torch)
    assert np.all(res["out"] == 0.0)
    ref_sel, _ = oracle.route(a["router_probs"], 2)
    np.testing.assert_array_equal(res["topk_idx"].reshape(6, 2), ref_sel)
    w2, b = W.random_case(rng, tokens_shape=(6,), hidden=64, experts=4, inter=32, k=2, bits=8, block_size=0,
                          activation="relu")
    b["input"] = b["input"][:0]
    b["router_probs"] = b["router_probs"][:0]
    res = run_gpu(b, w2.attrs(), torch, debug=False)
    assert res["out"].shape == (0, 64)


def test_error_statuses(torch):
    import quantized_mixture_experts_router_amd as qm
    rng = np.random.default_rng(84)
    w, a = W.random_case(rng, tokens_shape=(8,), hidden=64, experts=4, inter=32, k=2, bits=8, block_size=0,
                         activation="relu")
    d = {k: torch.from_numpy(v).cuda() for k, v in a.items()}
    args = [d[k] for k in ("input", "router_probs", "fc1_experts_weights", "fc1_scales", "fc2_experts_weights",
                           "fc2_scales")]
    need = qm.qmoe_workspace_size(*args, w.attrs())
    out = torch.full_like(d["input"], 5.0)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(qm.QmoeError) as ei:
        qm.qmoe_forward(*args, w.attrs(), out, small)
    assert ei.value.name == "WORKSPACE"
    big = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(qm.QmoeError) as ei:
        qm.qmoe_forward(*args, w.attrs(), out, big[4:])
    assert ei.value.name == "ALIGN"
    with pytest.raises(qm.QmoeError) as ei:
        qm.qmoe_forward(*args, dict(w.attrs(), k=9), out, big)
    assert ei.value.name == "ATTR"
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)  # untouched on error


# ------------------------------------------------------------------ full-size workloads
def _tile_tokens(counts, offsets, perm, k, bm=128):
    """Tokens whose slots fill whole M tiles of the tiled GEMMs: the first and
    the last (ragged) tile of every used expert, and every row of the expert
    with the fewest slots."""
    slots = []
    nz = np.nonzero(counts)[0]
    rare = nz[np.argmin(counts[nz])]
    for e in nz:
        lo, c = int(offsets[e]), int(counts[e])
        if e == rare:
            slots.append(perm[lo:lo + c])
            continue
        slots.append(perm[lo:lo + min(bm, c)])
        last = (c - 1) // bm * bm
        slots.append(perm[lo + last:lo + c])
    return sorted(set((np.concatenate(slots) // k).tolist()))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "prefill", "fine", "large_e"])
def test_full_size_workload(torch, name):
    w = W.WORKLOADS[name]
    say(f"[case] full {name}: generating")
    a = W.generate(w)
    attrs = w.attrs()
    res = run_gpu(a, attrs, torch)
    sel, wts = oracle.route(a["router_probs"], w.k)
    counts, offsets, perm = oracle.expert_permutation(sel, w.experts)
    check_routing(res, sel, wts, counts, offsets, perm)
    say(f"  routing bit-exact over {w.tokens} tokens; counts min/max {counts.min()}/{counts.max()}")
    out_all = res["out"].reshape(w.tokens, w.hidden)
    # every output row is written and finite (the output starts as NaN)
    assert np.all(np.isfinite(out_all)), f"{name}: {np.count_nonzero(~np.isfinite(out_all))} non-finite outputs"
    if name in ("decode", "fine"):
        ids = list(range(w.tokens))
    else:
        ids = _tile_tokens(counts, offsets, perm, w.k)
    say(f"  comparing {len(ids)} of {w.tokens} output rows with the oracle")
    ref = oracle.qmoe_tokens(ids, *a.values(), attrs=attrs)
    check_output(out_all[ids], ref, f"{name} ({len(ids)} rows)")
    # determinism at full size: bit-identical, and no NaN compares equal
    res2 = run_gpu(a, attrs, torch, debug=False)
    assert np.array_equal(res2["out"], res["out"], equal_nan=False)


def test_double_buffered_streaming(torch):
    """The streaming kernels' double-buffered mode (whole-K walks, several row
    blocks per workgroup, sized workgroups, fused activation), forced for
    every streaming GEMM: the decode workload in full and small shapes."""
    key = "QMOE_STREAM_SINGLE_STAGE_MAX_SPLITS"
    old = os.environ.get(key)
    os.environ[key] = "0"
    try:
        w = W.WORKLOADS["decode"]
        say("[case] decode, double-buffered streaming: generating")
        _full_check(w, W.generate(w), torch, "decode double-buffered")
        rng = np.random.default_rng(78)
        for bits in (4, 8):
            for bs, act in ((0, "relu"), (32, "swiglu"), (64, "swiglu")):
                for (T, H, E, I, k) in [(5, 128, 3, 64, 2), (16, 512, 8, 256, 2), (33, 256, 6, 128, 6),
                                        (64, 256, 4, 512, 2)]:
                    shape = (T,) if T % 2 else (2, T // 2)
                    wc, a = W.random_case(rng, tokens_shape=shape, hidden=H, experts=E, inter=I, k=k,
                                          bits=bits, block_size=bs, activation=act)
                    _full_check(wc, a, torch, f"double-buffered bits{bits} bs{bs} {act} T{T} H{H} E{E} I{I}")
    finally:
        if old is None:
            del os.environ[key]
        else:
            os.environ[key] = old


@pytest.mark.parametrize("tokens,bits,bs", [(16, 4, 64), (16, 8, 0), (200, 4, 32), (130, 8, 16)],
                         ids=["stream-int4", "stream-int8", "tiled-int4", "gemm-int8"])
def test_swiglu_limit(torch, tokens, bits, bs):
    # the clamp reading on every FC1 path: weight streaming (<= 96 tokens),
    # LDS-tiled, register-tiled (16-code blocks); limits that clamp a large
    # share of the FC1 values, and one above all of them
    rng = np.random.default_rng(40 + tokens + bits)
    w, a = W.random_case(rng, tokens_shape=(tokens,), hidden=256, experts=6, inter=128, k=2, bits=bits,
                         block_size=bs, activation="swiglu", scale_range=(0.01, 0.02))
    for lim, alpha, beta in ((0.05, 1.702, 1.0), (0.3, 1.0, 0.0), (1e30, 1.0, 0.0)):
        attrs = dict(w.attrs(), swiglu_limit=lim, activation_alpha=alpha, activation_beta=beta)
        label = f"limit={lim} T={tokens} bits={bits} bs={bs}"
        say(f"[case] {label}")
        res = run_gpu(a, attrs, torch)
        ref, inter = oracle.qmoe(*a.values(), attrs=attrs, return_intermediates=True)
        check_routing(res, inter["sel"], inter["w"], inter["counts"], inter["offsets"], inter["perm"])
        check_output(res["out"], ref, label)


@pytest.mark.parametrize("bs", [64, 128, 256])
@pytest.mark.parametrize("bits", [4, 8])
def test_tiled_scale_block_spans(torch, bs, bits):
    # the tiled kernels fold block sums once per span of one K step (64-code
    # blocks) or two K steps (128 codes and more); ragged expert tiles, both
    # activations, K of 6 or 10 K steps so that the six-step unroll leaves
    # a remainder
    rng = np.random.default_rng(500 + bs + bits)
    for act, (T, H, I) in (("swiglu", (200, 768, 256)), ("relu", (150, 512, 640))):
        if H % bs or I % bs:
            continue
        w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=5, inter=I, k=2, bits=bits, block_size=bs,
                             activation=act)
        _full_check(w, a, torch, f"tiled bs{bs} bits{bits} {act} T{T} H{H} I{I}")


# Segment scales between the tiled GEMMs: the FC1 epilogue writes FC2's hi/lo
# operand rows with one power-of-two scale per row tile and FC1 column tile;
# a row more than 2^12 below its tile's bound keeps its own exponent, which
# raises a flag, and FC2 then takes its rows back to one exponent each.
# (T, H, E, I, k, bits, bs, act, segments a row, FC1 scale factor per
# segment, extra attributes, decades of spread between token rows[, input
# scale])
SEGMENTS = [
    (300, 512, 4, 384, 2, 4, 128, "swiglu", 3, None, None, 0),
    (300, 512, 4, 640, 2, 4, 0, "relu", 3, None, None, 0),       # last FC1 column tile half empty
    (257, 1024, 6, 256, 2, 4, 256, "swiglu", 2, None, None, 0),
    (300, 512, 3, 512, 2, 4, 128, "swiglu", 4, (1e-4, 1e3, 1.0, 3e-2), None, 0),  # segments far apart
    (400, 256, 2, 256, 1, 4, 0, "relu", 1, (1e-6,), None, 0),
    (300, 512, 4, 320, 2, 4, 32, "swiglu", 3, None, None, 0),    # 32-code blocks, a partial column tile
    (300, 512, 4, 448, 2, 8, 64, "relu", 2, None, None, 0),
    (300, 512, 4, 384, 2, 8, 0, "swiglu", 3, (1e3, 1e-3, 1.0), None, 0),
    (260, 256, 3, 256, 2, 8, 128, "swiglu", 2, None, None, 0),
    (300, 512, 4, 384, 2, 4, 128, "swiglu", 3, None, dict(activation_alpha=1.702, activation_beta=1.0,
                                                          swiglu_limit=0.05), 0),
    (300, 512, 4, 384, 2, 4, 128, "swiglu", 3, None, None, 8),   # rows far apart: per-row exponents
    (300, 512, 4, 640, 2, 8, 0, "relu", 3, None, None, 8),
    (300, 512, 4, 320, 2, 4, 32, "relu", 2, None, None, 6),
    (300, 512, 4, 384, 2, 4, 128, "swiglu", 3, None, None, 0, 3e17),  # SwiGLU values past 2^113
]


@pytest.mark.parametrize("case", SEGMENTS)
def test_tiled_segment_scales(torch, monkeypatch, case):
    import re
    import quantized_mixture_experts_router_amd as qm
    T, H, E, I, k, bits, bs, act, nseg, factors, extra, spread = case[:12]
    xscale = case[12] if len(case) > 12 else 1.0
    rng = np.random.default_rng(1700 + T + I + bs + bits + spread)
    w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, bits=bits, block_size=bs,
                         activation=act)
    if factors:
        # FC1 columns of segment t (256 of them, the interleaved gate/linear
        # pairs of 128 codes with SwiGLU) scaled by factors[t]
        s1 = a["fc1_scales"].copy()
        for t, f in enumerate(factors):
            s1[:, 256 * t:256 * (t + 1)] *= np.float32(f)
        a["fc1_scales"] = s1
    if spread:
        a["input"] = (a["input"] * 10.0 ** rng.uniform(-spread, 0, size=(T, 1))).astype(np.float32)
    if xscale != 1.0:
        a["input"] = (a["input"].astype(np.float64) * xscale).astype(np.float32)
    attrs = dict(w.attrs(), **(extra or {}))
    label = (f"segments T{T} H{H} E{E} I{I} k{k} bits{bits} bs{bs} {act} factors={factors} {extra} spread={spread} "
             f"x{xscale:g}")
    for off in (False, True):
        # segment scales, then the per-row split between the GEMMs
        if off:
            monkeypatch.setenv("QMOE_TILED_SEGMENTS", "0")
        else:
            monkeypatch.delenv("QMOE_TILED_SEGMENTS", raising=False)
        plan = qm.qmoe_plan_describe(*a.values(), attrs=attrs)
        assert "fc1=tiled fc2=tiled" in plan and f"segments={0 if off else nseg} " in plan, plan
        say(f"[case] {label} {'per-row split' if off else ''}")
        res = run_gpu(a, attrs, torch, keep_ws=not off)
        ref, inter = oracle.qmoe(*a.values(), attrs=attrs, return_intermediates=True)
        check_routing(res, inter["sel"], inter["w"], inter["counts"], inter["offsets"], inter["perm"])
        assert np.all(np.isfinite(res["out"])), f"{label}: non-finite output"
        if spread or xscale != 1.0:
            # the bar per token row: a small row is held to its own magnitude
            out = res["out"].reshape(T, H).astype(np.float64)
            ref2 = np.asarray(ref, dtype=np.float64).reshape(T, H)
            err = np.max(np.abs(out - ref2), axis=1)
            rms = np.sqrt(np.mean(ref2 ** 2, axis=1))
            assert np.all(err <= OUT_TOL * rms), f"{label}: worst row {np.max(err / rms)}"
        else:
            check_output(res["out"], ref, label)
        if not off:
            # which FC2 ran: the flag FC1 raises for rows far below their tile
            at = int(re.search(r"segflag=(\d+)", plan).group(1))
            flag = int(res["ws"][at:at + 4].view(np.int32)[0])
            assert flag == (1 if spread or xscale > 1e16 else 0), f"{label}: flag {flag}"


# Half tiles (column-wise scales): each expert's last tile of at most 64
# rows runs as 64 rows x 512 columns (the second row of wavefronts takes the
# second 256 columns).  (T, H, E, I, k, bits, bs, act, logit bias of expert
# 0, extra environment): ragged expert counts, column-tile counts odd and
# even on both GEMMs (FC1 2I or I over 256, FC2 H / 256), both widths, with
# and without segment scales.
HALF_TILES = [
    (300, 768, 10, 384, 2, 4, 0, "swiglu", 0.0, {}),
    (300, 768, 10, 384, 2, 4, 0, "swiglu", 2.5, {"QMOE_TILED_SEGMENTS": "0"}),
    (280, 1280, 9, 640, 2, 8, 0, "relu", 0.0, {}),
    (333, 512, 16, 320, 3, 8, 0, "swiglu", 3.0, {}),
    (290, 256, 10, 256, 2, 8, 0, "swiglu", 0.0, {}),
    (400, 768, 7, 896, 1, 4, 0, "relu", 2.0, {"QMOE_TILED_SEGMENTS": "0"}),
]


@pytest.mark.parametrize("case", HALF_TILES)
def test_tiled_half_tiles(torch, monkeypatch, case):
    import quantized_mixture_experts_router_amd as qm
    T, H, E, I, k, bits, bs, act, bias, env = case
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    rng = np.random.default_rng(2100 + T + E + I + bits)
    w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, bits=bits, block_size=bs,
                         activation=act)
    # a bias makes expert 0 take several tiles (full ones, then a remainder)
    a["router_probs"] = a["router_probs"].copy()
    a["router_probs"][:, 0] += bias
    sel, _ = oracle.route(a["router_probs"], k)
    counts = np.bincount(sel.reshape(-1), minlength=E)
    small = int(np.sum((counts > 0) & (((counts - 1) % 128) < 64)))
    for off in (False, True):
        if off:
            monkeypatch.setenv("QMOE_TILED_HALF", "0")
        plan = qm.qmoe_plan_describe(*a.values(), attrs=w.attrs())
        assert "fc1=tiled fc2=tiled" in plan and f"half_tiles={0 if off else 1} " in plan, plan
        _full_check(w, a, torch, f"half tiles {'off' if off else 'on'} ({small} small tiles) T{T} H{H} E{E} I{I} "
                                 f"k{k} bits{bits} bs{bs} {act} bias{bias} {env}")


# K ranges of the tiled FC2 (a few tiles for 256 compute units): each range
# writes its own partial rows and the combine sums them in range order.
# (T, H, E, I, k, bits, bs, act, the plan's ranges, ranges forced through
# QMOE_TILED_KSPLIT, input spread in decades, extra environment): every
# scale layout the tiled kernel takes (blocks of 32 to 256 codes,
# column-wise with half tiles), two and four ranges of 256 codes and more,
# ReLU (256-code segments) and SwiGLU (128-code ones), rows flagged back to
# their own exponents (spread), and the per-row split between the GEMMs.
FC2_RANGES = [
    (300, 512, 4, 2048, 2, 4, 128, "swiglu", 2, (4, 1), 0, {}),
    (280, 512, 8, 2048, 2, 4, 32, "swiglu", 2, (4,), 0, {}),
    (260, 256, 4, 1536, 3, 4, 64, "relu", 1, (2,), 0, {}),
    (300, 512, 4, 2048, 2, 8, 256, "swiglu", 2, (4,), 0, {}),
    (300, 768, 6, 1024, 2, 8, 0, "relu", 1, (2, 4), 0, {}),
    (290, 256, 5, 4096, 2, 4, 0, "swiglu", 4, (1,), 0, {}),
    (300, 512, 4, 2048, 2, 4, 128, "swiglu", 2, (4,), 3, {}),
    (300, 512, 4, 2048, 2, 4, 128, "relu", 2, (4,), 0, {"QMOE_TILED_SEGMENTS": "0"}),
]


@pytest.mark.parametrize("case", FC2_RANGES)
def test_tiled_fc2_k_ranges(torch, monkeypatch, case):
    import quantized_mixture_experts_router_amd as qm
    T, H, E, I, k, bits, bs, act, ranges, forced, spread, env = case
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    rng = np.random.default_rng(2600 + T + E + I + bits + bs)
    w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, bits=bits, block_size=bs,
                         activation=act)
    if spread:
        a["input"] = (a["input"] * 10.0 ** rng.uniform(-spread, 0, size=(T, 1))).astype(np.float32)
    attrs = w.attrs()
    ref, inter = oracle.qmoe(*a.values(), attrs=attrs, return_intermediates=True)
    outs = []
    for ks in (None,) + tuple(forced):
        # the plan's own count, then the forced ones (a count whose ranges
        # would be under 256 codes leaves one range)
        if ks is None:
            monkeypatch.delenv("QMOE_TILED_KSPLIT", raising=False)
            want = ranges
        else:
            monkeypatch.setenv("QMOE_TILED_KSPLIT", str(ks))
            want = ks if I % (256 * ks) == 0 else 1
        plan = qm.qmoe_plan_describe(*a.values(), attrs=attrs)
        assert "fc1=tiled fc2=tiled" in plan and f"fc2_ranges={want} " in plan, plan
        label = f"FC2 ranges {want}: T{T} H{H} E{E} I{I} k{k} bits{bits} bs{bs} {act} spread={spread} {env}"
        say(f"[case] {label}")
        res = run_gpu(a, attrs, torch)
        check_routing(res, inter["sel"], inter["w"], inter["counts"], inter["offsets"], inter["perm"])
        assert np.all(np.isfinite(res["out"])), f"{label}: non-finite output"
        if spread:
            # the bar per token row: a small row is held to its own magnitude
            out = res["out"].reshape(T, H).astype(np.float64)
            ref2 = np.asarray(ref, dtype=np.float64).reshape(T, H)
            err = np.max(np.abs(out - ref2), axis=1)
            rms = np.sqrt(np.mean(ref2 ** 2, axis=1))
            assert np.all(err <= OUT_TOL * rms), f"{label}: worst row {np.max(err / rms)}"
        else:
            check_output(res["out"], ref, label)
        outs.append(res["out"].astype(np.float64))
    # the ranges split the same sums: the results agree to rounding
    ref_rms = np.sqrt(np.mean(np.asarray(ref, dtype=np.float64) ** 2))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-5 * ref_rms


@pytest.mark.parametrize("case", [
    # (T, H, E, I, k, bits, bs, act): one 16-row tile per expert with K-range
    # partials on the streaming path, many experts with tokens (dozens of
    # tiles, grids of several rounds), every scale layout the single-stage
    # kernel takes, and I = 1152 leaving a partial row block
    (16, 2048, 64, 1024, 8, 4, 64, "swiglu"),
    (16, 2048, 64, 1024, 8, 4, 0, "relu"),
    (10, 2048, 48, 1536, 6, 8, 32, "swiglu"),
    (7, 2048, 16, 2048, 2, 4, 256, "relu"),
    (12, 2048, 24, 1536, 5, 8, 128, "swiglu"),
    (16, 2048, 32, 1152, 4, 4, 128, "relu"),
])
def test_stream_many_experts(torch, case):
    T, H, E, I, k, bits, bs, act = case
    rng = np.random.default_rng(900 + T + E + bits)
    w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, bits=bits, block_size=bs,
                         activation=act)
    _full_check(w, a, torch, f"many experts T{T} H{H} E{E} I{I} k{k} bits{bits} bs{bs} {act}")


@pytest.mark.parametrize("case", [
    # (T, E, k, routing, normalize): the single-wavefront front end (T <= 64,
    # E * k <= 64) and the workgroup one beside it, with signed zeros and
    # repeated logits in every row
    (16, 8, 2, "qmoe", 0), (64, 64, 1, "qmoe", 0), (37, 16, 4, "moe", 0), (50, 32, 2, "moe", 1),
    (64, 8, 8, "qmoe", 0), (65, 8, 2, "qmoe", 0), (20, 40, 2, "moe", 0), (9, 64, 2, "qmoe", 0),
])
def test_front_end_ties_and_zeros(torch, case):
    T, E, k, routing, normalize = case
    rng = np.random.default_rng(77 + T + E + k)
    w = W.Workload("front", (T, 64), E, 32, k, 8, 0, "relu", (0.01, 0.02))
    a = W.generate(w, seed=int(rng.integers(0, 2**31 - 1)))
    # logits drawn from a few values (ties everywhere), with -0.0 and +0.0
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 2.0], dtype=np.float32)
    a["router_probs"] = vals[rng.integers(0, len(vals), size=(T, E))]
    attrs = dict(w.attrs(), routing=routing, normalize_routing_weights=normalize)
    res = run_gpu(a, attrs, torch)
    ref, inter = oracle.qmoe(*a.values(), attrs=attrs, return_intermediates=True)
    check_routing(res, inter["sel"], inter["w"], inter["counts"], inter["offsets"], inter["perm"],
                  selected_softmax=(routing == "qmoe" or normalize == 1))
    check_output(res["out"], ref, f"front end T{T} E{E} k{k} {routing}")


def test_two_streams_at_once(torch):
    # two calls in flight together on two streams, each with its own
    # workspace (the library keeps no per-call state of its own)
    import quantized_mixture_experts_router_amd as qm
    rng = np.random.default_rng(7100)
    cases = [W.random_case(rng, tokens_shape=(16,), hidden=2048, experts=8, inter=1024, k=2, bits=4, block_size=64,
                           activation="swiglu"),
             W.random_case(rng, tokens_shape=(180,), hidden=256, experts=6, inter=192, k=3, bits=8, block_size=0,
                           activation="relu")]
    names = ("input", "router_probs", "fc1_experts_weights", "fc1_scales", "fc2_experts_weights", "fc2_scales")
    runs = []
    for w, a in cases:
        args = [torch.from_numpy(np.ascontiguousarray(a[n])).cuda() for n in names]
        attrs = w.attrs()
        ws = torch.full((max(qm.qmoe_workspace_size(*args, attrs), 1),), 0xFF, dtype=torch.uint8, device="cuda")
        out = torch.full_like(args[0], float("nan"))
        runs.append((w, a, args, attrs, ws, out, torch.cuda.Stream()))
    torch.cuda.synchronize()
    for _ in range(3):
        for w, a, args, attrs, ws, out, st in runs:
            qm.qmoe_forward(*args, attrs, out, ws, st)
    torch.cuda.synchronize()
    for w, a, args, attrs, ws, out, st in runs:
        check_output(out.cpu().numpy(), oracle.qmoe(*[a[n] for n in names], attrs=attrs),
                     f"two streams T{w.tokens}")
