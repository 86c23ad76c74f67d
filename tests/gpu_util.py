"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle to the stated bar."""
import sys

import numpy as np

import quantized_mixture_experts_router_amd as qm

# Bars (stated before any kernel ran):
#   top-k indices, counts, offsets, permutation: bit-exact
#   routing weights: |gpu - oracle| <= 1e-6 * max(1, |oracle|)
#   output: max |gpu - oracle| <= 2e-3 * RMS(oracle output)
W_TOL = 1e-6
OUT_TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arrs, torch):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in arrs.items()}


def run_gpu(arrs, attrs, torch, debug=True, stream=None, keep_ws=False):
    """keep_ws: also return the workspace bytes after the call (res["ws"])."""
    d = to_dev(arrs, torch)
    T = int(np.prod(arrs["input"].shape[:-1]))
    E = arrs["fc1_experts_weights"].shape[0]  # experts the weights hold (counts/offsets are over them)
    k = attrs["k"]
    dbg = None
    if debug:
        dbg = dict(topk_idx=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
                   topk_w=torch.full((T * k,), -7.0, dtype=torch.float32, device="cuda"),
                   counts=torch.full((E,), -7, dtype=torch.int32, device="cuda"),
                   offsets=torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
                   perm=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"))
    out = torch.full_like(d["input"], float("nan"))
    # Workspace bytes 0xFF (every float a NaN): a read of anything the path
    # did not write first shows up in the output.
    args = [d[n] for n in ("input", "router_probs", "fc1_experts_weights", "fc1_scales", "fc2_experts_weights",
                           "fc2_scales")]
    need = qm.qmoe_workspace_size(*args, attrs)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    qm.forward(*args, attrs, output=out, debug=dbg, stream=stream, workspace=ws)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy()}
    if keep_ws:
        res["ws"] = ws.cpu().numpy()
    if dbg:
        res.update({kk: v.cpu().numpy() for kk, v in dbg.items()})
    return res


def check_routing(res, ref_sel, ref_w, ref_counts, ref_offsets, ref_perm, selected_softmax=True):
    """selected_softmax: the weights are a softmax over the k selected logits
    (QMoE routing, or MoE routing with renormalisation), so k = 1 gives 1.0."""
    T, k = ref_sel.shape
    np.testing.assert_array_equal(res["topk_idx"].reshape(T, k), ref_sel)
    err = np.abs(res["topk_w"].reshape(T, k).astype(np.float64) - ref_w)
    assert np.all(err <= W_TOL * np.maximum(1.0, np.abs(ref_w))), float(err.max())
    if k == 1 and selected_softmax:
        assert np.all(res["topk_w"] == np.float32(1.0))
    np.testing.assert_array_equal(res["counts"], ref_counts)
    np.testing.assert_array_equal(res["offsets"], ref_offsets)
    np.testing.assert_array_equal(res["perm"], ref_perm)


def check_output(out, ref, label=""):
    ref = np.asarray(ref, dtype=np.float64).reshape(out.shape)
    assert np.all(np.isfinite(out)), f"{label}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(out.astype(np.float64) - ref))) if ref.size else 0.0
    say(f"  {label}: max|err| = {err:.3e}, rms(ref) = {rms:.3e}, ratio = {err / rms if rms else 0:.3e}")
    assert err <= OUT_TOL * rms or (rms == 0 and err == 0), f"{label}: {err} > {OUT_TOL} * {rms}"
    return err, rms
