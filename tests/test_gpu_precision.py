"""GPU parity over the magnitude range of the float32 input contract.

The matrix cores take f16 operands: every fp32 operand row (the layer input
for FC1, the activation rows for FC2) is scaled by a power of two of its own
and split into f16 hi + lo.  These cases run each GEMM path (weight streaming
in its single-stage and double-buffered modes, the LDS-tiled GEMM and the
register-tiled one) on inputs far below and far above the f16 range, and on
rows whose magnitudes differ by many orders, against the float64 oracle.

Bar: routing bit-exact; output max-abs error <= 2e-3 x RMS of the oracle's
output, checked per token row (so a small row is held to its own magnitude,
not to the largest row's).
"""
import os
import zlib

import numpy as np
import pytest

import oracle
from quantized_mixture_experts_router_amd import workloads as W

from gpu_util import OUT_TOL, check_routing, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


# (label, T, H, E, I, k, bits, bs, env): one case per GEMM path
PATHS = [
    ("stream", 16, 512, 6, 256, 2, 4, 64, None),
    ("stream-int8", 24, 512, 6, 256, 2, 8, 0, None),
    ("stream-double-buffered", 16, 512, 6, 256, 2, 4, 64, "0"),
    ("tiled", 200, 256, 5, 192, 2, 4, 32, None),
    ("tiled-int8", 150, 384, 4, 128, 3, 8, 0, None),
    ("gemm", 130, 256, 4, 128, 2, 8, 16, None),
]


def check_rows(out, ref, label):
    """Per token row: max |gpu - oracle| <= OUT_TOL * RMS(oracle row)."""
    out = out.reshape(ref.shape).astype(np.float64)
    assert np.all(np.isfinite(out)), f"{label}: non-finite output"
    err = np.max(np.abs(out - ref), axis=1)
    rms = np.sqrt(np.mean(ref ** 2, axis=1))
    zero = rms == 0
    assert np.all(err[zero] == 0), f"{label}: nonzero output where the oracle's row is zero"
    ratio = err[~zero] / rms[~zero]
    say(f"  {label}: worst row max|err|/rms = {ratio.max():.3e} over {(~zero).sum()} rows "
        f"(row rms {rms[~zero].min():.3e} .. {rms[~zero].max():.3e})")
    assert np.all(ratio <= OUT_TOL), f"{label}: {ratio.max()} > {OUT_TOL}"


def _run(torch, path, act, x_transform, seed):
    label, T, H, E, I, k, bits, bs, env = path
    rng = np.random.default_rng(seed)
    w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, bits=bits, block_size=bs,
                         activation=act)
    a["input"] = x_transform(a["input"], rng).astype(np.float32)
    key = "QMOE_STREAM_SINGLE_STAGE_MAX_SPLITS"
    old = os.environ.get(key)
    if env is not None:
        os.environ[key] = env
    try:
        res = run_gpu(a, w.attrs(), torch)
    finally:
        if env is not None:
            if old is None:
                del os.environ[key]
            else:
                os.environ[key] = old
    ref, inter = oracle.qmoe(*a.values(), attrs=w.attrs(), return_intermediates=True)
    check_routing(res, inter["sel"], inter["w"], inter["counts"], inter["offsets"], inter["perm"])
    return res["out"], np.asarray(ref, dtype=np.float64).reshape(T, H)


@pytest.mark.parametrize("scale", [1e-7, 1e-5, 1e-3, 1e3, 1e5], ids=lambda s: f"x{s:g}")
@pytest.mark.parametrize("act", ["relu", "swiglu"])
@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
def test_input_scaled(torch, path, act, scale):
    # the whole input scaled: below the f16 normal range (6.1e-5), below its
    # subnormal range (6e-8), and above its largest value (65504)
    say(f"[case] {path[0]} {act} input x{scale:g}")
    out, ref = _run(torch, path, act, lambda x, rng: x.astype(np.float64) * scale, 3000 + zlib.crc32(f"{path[0]}:{act}".encode()) % 1000)
    check_rows(out, ref, f"{path[0]} {act} x{scale:g}")


@pytest.mark.parametrize("act", ["relu", "swiglu"])
@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
def test_rows_of_different_magnitudes(torch, path, act):
    # every token row scaled by its own 10^U(-8, 4), and inside rows single
    # elements by 10^U(-6, 0): one call holds rows (and FC2 operand rows)
    # many orders of magnitude apart
    def tr(x, rng):
        x = x.astype(np.float64)
        x *= 10.0 ** rng.uniform(-8, 4, size=(x.shape[0], 1))
        x *= 10.0 ** rng.uniform(-6, 0, size=x.shape)
        return x
    say(f"[case] {path[0]} {act} rows of different magnitudes")
    out, ref = _run(torch, path, act, tr, 4000 + zlib.crc32(f"{path[0]}:{act}".encode()) % 1000)
    check_rows(out, ref, f"{path[0]} {act} mixed rows")
