"""GPU parity of GroupedMatMul (ONNX "GroupedMatMul - 29") through the C ABI.

Bar (float32 products and sums, stated before the kernel ran): every output
element within 2 (K + 1) 2^-24 (sum_c |x[m, c] w[g, c, n]| + |bias[g, n]|) of
the float64 oracle, twice the worst-case rounding bound of a float32 sum of
K + 1 terms in any order.  Rows whose index lies outside [0, G) (the page
leaves them undefined) must be zero, the library's stated choice.
Small cases compare every element; the full-size workloads compare sampled
rows that the oracle computes one by one.
"""
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

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _bound(x, w, idx, bias, rows):
    """Per-element error bar for the selected rows (float64)."""
    K = x.shape[1]
    ax = np.abs(x[rows].astype(np.float64))
    out = np.empty((len(rows), idx.shape[1], w.shape[2]))
    for r, m in enumerate(rows):
        for i in range(idx.shape[1]):
            g = int(idx[m, i])
            out[r, i] = ax[r] @ np.abs(w[g].astype(np.float64))
            if bias is not None:
                out[r, i] += abs(bias[g].astype(np.float64))
    return 2.0 * (K + 1) * U32 * out + 1e-30


def _run(torch, x, w, idx, bias, misalign=False, label=""):
    """GroupedMatMul on the GPU; output pre-filled with NaN, workspace with 0xFF."""
    def dev(a, off=0):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        if not off:
            return t.cuda()
        buf = torch.empty(t.numel() + off, dtype=t.dtype, device="cuda")
        v = buf[off:].view(t.shape)
        v.copy_(t.cuda())
        return v
    off = 1 if misalign else 0
    dx, dw, di, db = dev(x, off), dev(w, off), dev(idx), dev(bias)
    M, S, N = x.shape[0], idx.shape[1], w.shape[2]
    out = torch.full((M, S, N), float("nan"), dtype=torch.float32, device="cuda")
    need = qm.qmoe_grouped_matmul_workspace_size(dx, dw, di, db, out)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    say(f"[gmm] {label} M={M} K={x.shape[1]} G={w.shape[0]} N={N} S={S} bias={bias is not None} "
        f"idx={idx.dtype} misalign={misalign} ws={need}")
    qm.qmoe_grouped_matmul(dx, dw, di, db, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(got, x, w, idx, bias, rows=None, label=""):
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    G = w.shape[0]
    valid = (idx >= 0) & (idx < G)
    sub = got[rows]
    assert not np.isnan(sub).any(), f"{label}: unwritten output"
    vi = np.where(valid, idx, 0)
    ref = oracle.grouped_matmul_rows(x, w, vi, bias, rows)
    bar = _bound(x, w, vi, bias, rows)
    ok = valid[rows][:, :, None]
    err = np.where(ok, np.abs(sub.astype(np.float64) - ref), 0.0)
    worst = float((err / bar).max()) if err.size else 0.0
    say(f"[gmm] {label} max err / bar = {worst:.3g}")
    assert np.all(err <= bar), f"{label}: max err/bar {worst}"
    # rows with an invalid index are zero
    assert np.all(np.where(ok, 0.0, sub) == 0.0), f"{label}: invalid-index rows not zero"


def _golden():
    with open(os.path.join(GOLDEN, "grouped_matmul_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_page_examples(torch, case):
    inp = np.array(case["input"], dtype=np.float32)
    if "input_shape" in case:
        inp = inp.reshape(case["input_shape"])
    wts = np.array(case["weights"], dtype=np.float32)
    for it in (np.int32, np.int64):
        idx = np.array(case["group_indices"], dtype=it)
        if "group_indices_shape" in case:
            idx = idx.reshape(case["group_indices_shape"])
        elif idx.size == 0:
            idx = idx.reshape(inp.shape[0], 0)
        bias = None if case["bias"] is None else np.array(case["bias"], dtype=np.float32)
        got = _run(torch, inp, wts, idx, bias, label=case["name"])
        assert got.shape == tuple(case["expected_shape"])
        if case["expected"] is not None:
            # float32 of the page's values: integers exact, x.y within one rounding
            np.testing.assert_allclose(got, np.array(case["expected"]), rtol=2 * U32, atol=0)


SHAPES = [  # M, K, G, N, S: one tile, several tiles, ragged K / N / M tails
    # at most 16 rows per group on average, K and N multiples of 4: 16-row
    # tiles, weight-streaming kernel
    (16, 256, 8, 512, 2),
    (20, 100, 16, 260, 3),
    (8, 8, 4, 64, 2),
    (8, 4, 4, 68, 2),
    # 64-row tiles, LDS-tiled kernel
    (1, 1, 1, 1, 1),
    (5, 3, 2, 7, 2),
    (64, 16, 1, 128, 1),
    (100, 64, 4, 200, 3),
    (257, 96, 3, 384, 1),
    (300, 130, 7, 257, 2),
    (129, 260, 5, 132, 4),
    (33, 1000, 9, 96, 3),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_random_shapes(torch, shape):
    M, K, G, N, S = shape
    for seed, (bias_on, it) in enumerate([(True, np.int64), (False, np.int32)]):
        rng = np.random.default_rng(100 + seed + 7 * M)
        x = rng.standard_normal((M, K), dtype=np.float32)
        w = rng.standard_normal((G, K, N), dtype=np.float32)
        b = rng.standard_normal((G, N), dtype=np.float32) if bias_on else None
        idx = rng.integers(0, G, size=(M, S)).astype(it)
        got = _run(torch, x, w, idx, b, label=f"rand{shape}")
        _check(got, x, w, idx, b, label=f"rand{shape}")


def test_skewed_and_unused_groups(torch):
    # most rows in one group (several tiles of it), some groups never used,
    # repeated selections of one group within a row
    rng = np.random.default_rng(7)
    M, K, G, N, S = 400, 128, 12, 256, 3
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((G, K, N), dtype=np.float32)
    b = rng.standard_normal((G, N), dtype=np.float32)
    idx = np.where(rng.random((M, S)) < 0.8, 5, rng.choice([0, 11, 3], size=(M, S))).astype(np.int64)
    got = _run(torch, x, w, idx, b, label="skewed")
    _check(got, x, w, idx, b, label="skewed")


@pytest.mark.parametrize("shape", [(70, 64, 3, 136, 2), (16, 64, 8, 136, 2)], ids=["tiles64", "tiles16"])
def test_misaligned_pointers_take_scalar_path(torch, shape):
    # input and weights 4 bytes past a 16-byte boundary: scalar loads, and
    # 16-row tiles run on the LDS-tiled kernel
    rng = np.random.default_rng(8)
    M, K, G, N, S = shape
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((G, K, N), dtype=np.float32)
    b = rng.standard_normal((G, N), dtype=np.float32)
    idx = rng.integers(0, G, size=(M, S))
    got = _run(torch, x, w, idx, b, misalign=True, label="misaligned")
    _check(got, x, w, idx, b, label="misaligned")


def test_streaming_one_strip_per_wavefront_with_tails(torch):
    # enough 256-column blocks that the streaming kernel gives each
    # wavefront its own column strip (no K split); N % 256 != 0, K % 16 != 0
    rng = np.random.default_rng(13)
    M, K, G, N, S = 16, 100, 8, 20004, 1
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((G, K, N), dtype=np.float32)
    b = rng.standard_normal((G, N), dtype=np.float32)
    idx = rng.permutation(np.repeat(np.arange(G), 2))[:, None]
    got = _run(torch, x, w, idx, b, label="rows16-strips")
    _check(got, x, w, idx, b, label="rows16-strips")


def test_small_groups_spanning_several_16_row_tiles(torch):
    # 16-row tiles with one group of 40 rows (three tiles) and a few empty groups
    rng = np.random.default_rng(12)
    M, K, G, N, S = 64, 64, 8, 128, 1
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((G, K, N), dtype=np.float32)
    b = rng.standard_normal((G, N), dtype=np.float32)
    idx = np.concatenate([np.zeros(40, np.int64), rng.choice([2, 5, 7], size=M - 40)])[:, None]
    got = _run(torch, x, w, idx, b, label="rows16-multi")
    _check(got, x, w, idx, b, label="rows16-multi")


@pytest.mark.parametrize("shape", [(150, 48, 4, 160, 3), (16, 64, 4, 128, 2)], ids=["tiles64", "tiles16"])
def test_invalid_indices_give_zero_rows(torch, shape):
    rng = np.random.default_rng(9)
    M, K, G, N, S = shape
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((G, K, N), dtype=np.float32)
    b = rng.standard_normal((G, N), dtype=np.float32)
    for it in (np.int32, np.int64):
        idx = rng.integers(0, G, size=(M, S)).astype(it)
        bad = rng.random((M, S)) < 0.2
        vals = np.array([-1, G, G + 5, -G, np.iinfo(it).max, np.iinfo(it).min], dtype=it)
        idx[bad] = rng.choice(vals, size=int(bad.sum()))
        got = _run(torch, x, w, idx, b, label=f"invalid-{np.dtype(it).name}")
        _check(got, x, w, idx, b, label=f"invalid-{np.dtype(it).name}")


def test_degenerate_sizes(torch):
    rng = np.random.default_rng(10)
    # K == 0: the bias alone (or zeros)
    b = rng.standard_normal((3, 20), dtype=np.float32)
    idx = rng.integers(0, 3, size=(9, 2))
    got = _run(torch, np.zeros((9, 0), np.float32), np.zeros((3, 0, 20), np.float32), idx, b, label="K0")
    np.testing.assert_array_equal(got, b[idx])
    got = _run(torch, np.zeros((9, 0), np.float32), np.zeros((3, 0, 20), np.float32), idx, None, label="K0-nobias")
    np.testing.assert_array_equal(got, np.zeros_like(got))
    # G == 0: every index is invalid -> zeros
    got = _run(torch, rng.standard_normal((6, 8), dtype=np.float32), np.zeros((0, 8, 12), np.float32),
               np.zeros((6, 2), np.int64), None, label="G0")
    np.testing.assert_array_equal(got, np.zeros((6, 2, 12)))
    # M, S or N == 0: empty output, nothing enqueued
    for (M, S, N) in ((0, 2, 5), (4, 0, 5), (4, 2, 0)):
        got = _run(torch, np.ones((M, 3), np.float32), np.ones((2, 3, N), np.float32),
                   np.zeros((M, S), np.int64), None, label=f"empty{(M, S, N)}")
        assert got.shape == (M, S, N)


@pytest.mark.parametrize("name", sorted(n for n, w in W.GMM_WORKLOADS.items() if w.dtype == "float32"))
def test_full_size_workloads_sampled(torch, name):
    w = W.GMM_WORKLOADS[name]
    a = W.gmm_generate(w)
    got = _run(torch, a["input"], a["weights"], a["group_indices"], a["bias"], label=name)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, size=min(w.M, 10), replace=False)]))
    _check(got, a["input"], a["weights"], a["group_indices"], a["bias"], rows=rows, label=name)
    # every element written, and finite
    assert np.isfinite(got).all()
