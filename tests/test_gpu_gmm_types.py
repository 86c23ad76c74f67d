"""GPU parity of GroupedMatMul (ONNX "GroupedMatMul - 29") in the page's
other floating types: float16, bfloat16 and double (Type Constraints).

Bars, per output element, stated before the kernels ran (ref = the float64
oracle on the same typed inputs, A = sum_c |x[m, c] w[g, c, n]| + |bias|):
  float16:  |gpu - ref| <= 2^-11 (|ref| + e32) + 2^-25 + e32
  bfloat16: |gpu - ref| <= 2^-8 (|ref| + e32) + e32
  double:   |gpu - ref| <= 2 (K + 1) 2^-53 A
with e32 = 2 (K + 1) 2^-24 A: the products of 16-bit values are exact, the
float32 sum of K + 1 terms errs by at most e32/2, and the one rounding to
the output type by half a unit in its last place (2^-11 or 2^-8 relative
for normal results; 2^-25 absolute below the float16 normal range).
Rows with an index outside [0, G) must be zero (the library's choice).
"""
import functools
import json
import os

import numpy as np
import pytest

import oracle
import quantized_mixture_experts_router_amd as qm
from quantized_mixture_experts_router_amd import workloads as W

from conftest import GOLDEN
from gpu_util import say

pytestmark = pytest.mark.gpu

TYPES = ["float16", "bfloat16", "float64"]


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _typed(torch, a, dt):
    """A float array as a torch tensor of type dt (round to nearest even), and
    its exact float64 values."""
    if a is None:
        return None, None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(getattr(torch, dt))
    return t, t.to(torch.float64).numpy()


def _run(torch, x, w, idx, bias, dt, misalign=False, label=""):
    """GroupedMatMul in type dt on the GPU (output pre-filled with NaN,
    workspace with 0xFF); returns (output as float64, typed inputs as float64)."""
    tx, fx = _typed(torch, x, dt)
    tw, fw = _typed(torch, w, dt)
    tb, fb = _typed(torch, bias, dt)

    def dev(t, off=0):
        if t is None:
            return None
        if not off:
            return t.cuda()
        buf = torch.empty(t.numel() + off, dtype=t.dtype, device="cuda")
        v = buf[off:].view(t.shape)
        v.copy_(t.cuda())
        return v
    off = int(misalign)  # elements: True = 1
    dx, dw, db = dev(tx, off), dev(tw, off), dev(tb)
    di = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    M, S, N = x.shape[0], idx.shape[1], w.shape[2]
    out = torch.full((M, S, N), float("nan"), dtype=getattr(torch, dt), device="cuda")
    need = qm.qmoe_grouped_matmul_workspace_size(dx, dw, di, db, out)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    say(f"[gmm-{dt}] {label} M={M} K={x.shape[1]} G={w.shape[0]} N={N} S={S} bias={bias is not None} "
        f"idx={idx.dtype} misalign={misalign}")
    qm.qmoe_grouped_matmul(dx, dw, di, db, out, ws)
    torch.cuda.synchronize()
    return out.to(torch.float64).cpu().numpy(), fx, fw, fb


def _bar(dt, ref, A, K):
    e32 = 2.0 * (K + 1) * 2.0 ** -24 * A
    if dt == "float16":
        return 2.0 ** -11 * (np.abs(ref) + e32) + 2.0 ** -25 + e32
    if dt == "bfloat16":
        return 2.0 ** -8 * (np.abs(ref) + e32) + e32
    return 2.0 * (K + 1) * 2.0 ** -53 * A + 1e-300


def _check(dt, got, x, w, idx, bias, rows=None, label=""):
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    G, K = w.shape[0], x.shape[1]
    valid = (idx >= 0) & (idx < G)
    sub = got[rows]
    assert not np.isnan(sub).any(), f"{label}: unwritten output"
    vi = np.where(valid, idx, 0)
    ref = oracle.grouped_matmul_rows(x, w, vi, bias, rows)
    A = oracle.grouped_matmul_rows(np.abs(x), np.abs(w), vi, None if bias is None else np.abs(bias), rows)
    bar = _bar(dt, ref, A, K)
    ok = valid[rows][:, :, None]
    err = np.where(ok, np.abs(sub - ref), 0.0)
    worst = float((err / bar).max()) if err.size else 0.0
    say(f"[gmm-{dt}] {label} max err / bar = {worst:.3g}")
    assert np.all(err <= bar), f"{label}: max err/bar {worst}"
    assert np.all(np.where(ok, 0.0, sub) == 0.0), f"{label}: invalid-index rows not zero"


def _additional_types_case():
    with open(os.path.join(GOLDEN, "grouped_matmul_examples.json")) as f:
        return next(c for c in json.load(f)["cases"] if c["name"] == "additional_types")


@pytest.mark.parametrize("dt", TYPES)
def test_page_additional_types_example(torch, dt):
    # the page's float16 / float64 example (Examples, _additional_types), with
    # int32 and int64 indices; its values are exact in bfloat16 too
    c = _additional_types_case()
    assert dt in c["dtypes"] or dt == "bfloat16"
    for it in c["index_dtypes"]:
        got, *_ = _run(torch, np.array(c["input"], np.float64), np.array(c["weights"], np.float64),
                       np.array(c["group_indices"], dtype=it), np.array(c["bias"], np.float64), dt,
                       label=f"additional_types idx {it}")
        assert got.shape == tuple(c["expected_shape"])
        np.testing.assert_array_equal(got, np.array(c["expected"]))


SHAPES = [  # M, K, G, N, S: one tile, several tiles, ragged K / N / M tails
    (1, 1, 1, 1, 1), (5, 3, 2, 7, 2), (16, 256, 8, 512, 2), (64, 32, 1, 128, 1), (100, 64, 4, 200, 3),
    (257, 96, 3, 384, 1), (300, 130, 7, 257, 2), (129, 260, 5, 132, 4), (33, 1000, 9, 96, 3),
    (200, 1000, 3, 136, 2),
]


@pytest.mark.parametrize("dt", TYPES)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_random_shapes(torch, shape, dt):
    M, K, G, N, S = shape
    for seed, (bias_on, it) in enumerate([(True, np.int64), (False, np.int32)]):
        rng = np.random.default_rng(300 + seed + 7 * M + K)
        x = rng.standard_normal((M, K))
        w = rng.standard_normal((G, K, N)) * 0.1
        b = rng.standard_normal((G, N)) if bias_on else None
        idx = rng.integers(0, G, size=(M, S)).astype(it)
        got, fx, fw, fb = _run(torch, x, w, idx, b, dt, label=f"rand{shape}")
        _check(dt, got, fx, fw, idx, fb, label=f"rand{shape}")


@pytest.mark.parametrize("dt", TYPES)
def test_invalid_indices_misaligned_and_empty(torch, dt):
    rng = np.random.default_rng(31)
    M, K, G, N, S = 150, 48, 4, 160, 3
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((G, K, N)) * 0.1
    b = rng.standard_normal((G, N))
    for it in (np.int32, np.int64):
        idx = rng.integers(0, G, size=(M, S)).astype(it)
        bad = rng.random((M, S)) < 0.2
        vals = np.array([-1, G, G + 5, np.iinfo(it).max, np.iinfo(it).min], dtype=it)
        idx[bad] = rng.choice(vals, size=int(bad.sum()))
        got, fx, fw, fb = _run(torch, x, w, idx, b, dt, label=f"invalid-{np.dtype(it).name}")
        _check(dt, got, fx, fw, idx, fb, label=f"invalid-{np.dtype(it).name}")
    # input and weights one element past a 16-byte boundary: scalar loads
    idx = rng.integers(0, G, size=(M, S))
    got, fx, fw, fb = _run(torch, x, w, idx, b, dt, misalign=True, label="misaligned")
    _check(dt, got, fx, fw, idx, fb, label="misaligned")
    # K == 0: the bias alone
    idx = rng.integers(0, G, size=(9, 2))
    got, _, _, fb = _run(torch, np.zeros((9, 0)), np.zeros((G, 0, N)), idx, b, dt, label="K0")
    np.testing.assert_array_equal(got, fb[idx])


@pytest.mark.parametrize("dt", ["float16", "bfloat16"])
@pytest.mark.parametrize("tile_rows", ["64", "128"])
def test_tile_rows_choices(torch, dt, tile_rows, monkeypatch):
    # the 16-bit tile kernel on 64- and 128-row tiles (the library picks by
    # rows per group; the variable forces either): ragged M, K and N tails,
    # invalid indices, one group with most of the rows
    monkeypatch.setenv("QMOE_GMM16_TILE_ROWS", tile_rows)
    rng = np.random.default_rng(41)
    for M, K, G, N, S in [(257, 96, 3, 384, 1), (300, 200, 5, 136, 2), (40, 520, 2, 264, 4)]:
        x = rng.standard_normal((M, K))
        w = rng.standard_normal((G, K, N)) * 0.1
        b = rng.standard_normal((G, N))
        idx = np.where(rng.random((M, S)) < 0.6, 0, rng.integers(0, G, size=(M, S))).astype(np.int64)
        idx[rng.random((M, S)) < 0.1] = G + 2
        label = f"rows{tile_rows}-{M}x{K}x{G}x{N}x{S}"
        got, fx, fw, fb = _run(torch, x, w, idx, b, dt, label=label)
        _check(dt, got, fx, fw, idx, fb, label=label)


@pytest.mark.parametrize("dt", TYPES)
def test_streaming_variants(torch, dt):
    # groups of at most 16 rows take the weight-streaming kernels: the 16-bit
    # matrix-instruction one (K, N multiples of 8, 16-byte aligned), with and
    # without K ranges, the widening one (K or N only multiples of 4, or
    # 8-byte aligned), the double one (N even, 16-byte aligned); ragged K
    # groups, invalid indices
    rng = np.random.default_rng(43)
    cases = [((24, 260, 6, 132, 2), 0), ((16, 64, 16, 16384, 2), 0), ((16, 264, 8, 256, 2), 4),
             ((20, 1000, 4, 520, 3), 0), ((18, 72, 3, 136, 2), 0)]
    for (M, K, G, N, S), off in cases:
        x = rng.standard_normal((M, K))
        w = rng.standard_normal((G, K, N)) * 0.1
        b = rng.standard_normal((G, N))
        idx = rng.integers(0, G, size=(M, S)).astype(np.int64)
        idx[rng.random((M, S)) < 0.15] = -3
        label = f"stream-{M}x{K}x{G}x{N}x{S}-off{off}"
        got, fx, fw, fb = _run(torch, x, w, idx, b, dt, misalign=off, label=label)
        _check(dt, got, fx, fw, idx, fb, label=label)


@functools.lru_cache(maxsize=1)
def _decode_case():
    # drawn once for the three types (940 M weights)
    return W.gmm_generate(W.GMM_WORKLOADS["gmm_decode_fc1"])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dt", TYPES)
def test_decode_workload_sampled(torch, dt):
    # the decode layer's FC1 as a GroupedMatMul (16 x 4096 -> 28672, 8 groups,
    # 2 a row): the weight slices of every used group once, inputs rounded to
    # the type
    w = W.GMM_WORKLOADS["gmm_decode_fc1"]
    a = _decode_case()
    got, fx, fw, fb = _run(torch, a["input"], a["weights"], a["group_indices"], a["bias"], dt, label=w.name)
    assert np.isfinite(got).all()
    _check(dt, got, fx, fw, a["group_indices"], fb, rows=np.arange(w.M), label=w.name)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dt", TYPES)
def test_fine_grained_workload_sampled(torch, dt):
    # the fine-grained layer's FC1 as a GroupedMatMul (2048 x 2048 -> 2816,
    # 64 groups, 6 a row, skewed), inputs rounded to the type
    w = W.GMM_WORKLOADS["gmm_fine_fc1"]
    a = W.gmm_generate(w)
    got, fx, fw, fb = _run(torch, a["input"], a["weights"], a["group_indices"], a["bias"], dt, label=w.name)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(32)
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, size=12, replace=False)]))
    _check(dt, got, fx, fw, a["group_indices"], fb, rows=rows, label=w.name)
