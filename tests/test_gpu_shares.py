"""GPU parity of one GPU's shares of the operator (no collectives: the part
of an expert-parallel or inter-size-parallel layer that one GPU computes).

* Expert shares (attribute first_expert): the weights hold a range of the
  router's experts; routing over all E logits is bit-exact, counts, offsets
  and the permutation (held experts' slots first, stable, then the others)
  are bit-exact against the oracle's share, outputs within 2e-3 x RMS; the
  shares of a partition, computed on the GPU, sum to the oracle's whole
  output.  Every GEMM path: weight streaming, LDS-tiled, register-tiled.
* The expert share of the 128-expert layer at full size (16 experts from
  expert 0 with that layer's routing), and the decode layer with its inter
  size split 8 ways, at full size.
"""
import numpy as np
import pytest

import oracle
from quantized_mixture_experts_router_amd import workloads as W

from gpu_util import check_output, check_routing, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _expert_share(a, first, held):
    b = dict(a)
    for n in ("fc1_experts_weights", "fc1_scales", "fc2_experts_weights", "fc2_scales"):
        b[n] = np.ascontiguousarray(a[n][first:first + held])
    return b


CASES = [
    # (T, H, E, I, k, bits, bs, act, cuts, environment): one case per GEMM
    # path, and the LDS-tiled FC2 in four K ranges (partial sets of the held
    # slots only)
    (16, 512, 8, 256, 2, 4, 64, "swiglu", [0, 3, 4, 8], {}),        # weight streaming
    (40, 256, 12, 128, 3, 8, 0, "relu", [0, 5, 12], {}),            # weight streaming, int8
    (200, 256, 8, 192, 2, 4, 32, "swiglu", [0, 1, 6, 8], {}),       # LDS-tiled
    (130, 256, 6, 128, 2, 8, 16, "relu", [0, 2, 6], {}),            # register-tiled (16-code blocks)
    (300, 256, 8, 2048, 2, 4, 128, "swiglu", [0, 3, 8], {"QMOE_TILED_KSPLIT": "4"}),  # tiled, FC2 ranges
]


@pytest.mark.parametrize("case", CASES, ids=["stream", "stream-int8", "tiled", "gemm", "tiled-fc2-ranges"])
def test_expert_shares(torch, monkeypatch, case):
    T, H, E, I, k, bits, bs, act, cuts, env = case
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    rng = np.random.default_rng(800 + T + E)
    w, a = W.random_case(rng, tokens_shape=(T,), hidden=H, experts=E, inter=I, k=k, bits=bits, block_size=bs,
                         activation=act)
    total = np.zeros((T, H))
    for first, last in zip(cuts[:-1], cuts[1:]):
        b = _expert_share(a, first, last - first)
        attrs = dict(w.attrs(), first_expert=first)
        label = f"share [{first}, {last}) of {E} T{T} bits{bits} bs{bs} {act}"
        say(f"[case] {label} {env}")
        res = run_gpu(b, attrs, torch)
        ref, inter = oracle.qmoe(*b.values(), attrs=attrs, return_intermediates=True)
        check_routing(res, inter["sel"], inter["w"], inter["counts"], inter["offsets"], inter["perm"])
        check_output(res["out"], ref, label)
        total += res["out"].astype(np.float64).reshape(T, H)
    full = oracle.qmoe(*a.values(), attrs=w.attrs()).reshape(T, H)
    check_output(total, full, f"sum of the shares vs the whole operator T{T}")


def test_share_without_experts_and_bad_range(torch):
    import quantized_mixture_experts_router_amd as qm
    rng = np.random.default_rng(820)
    w, a = W.random_case(rng, tokens_shape=(10,), hidden=64, experts=4, inter=64, k=2, bits=8, block_size=0,
                         activation="relu")
    b = _expert_share(a, 2, 0)
    res = run_gpu(b, dict(w.attrs(), first_expert=2), torch)
    assert np.all(res["out"] == 0.0)
    sel, _ = oracle.route(a["router_probs"], 2)
    np.testing.assert_array_equal(res["topk_idx"].reshape(10, 2), sel)
    b = _expert_share(a, 1, 2)
    d = {n: torch.from_numpy(np.ascontiguousarray(v)).cuda() for n, v in b.items()}
    args = [d[n] for n in ("input", "router_probs", "fc1_experts_weights", "fc1_scales", "fc2_experts_weights",
                           "fc2_scales")]
    out = torch.full_like(d["input"], 5.0)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(qm.QmoeError) as ei:
        qm.qmoe_forward(*args, dict(w.attrs(), first_expert=3), out, ws)
    assert ei.value.name == "ATTR"
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)


def _tile_tokens(counts, offsets, perm, k, bm=128):
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
@pytest.mark.parametrize("name", ["large_e_ep8", "decode_tp8"])
def test_full_size_share(torch, name):
    w = W.WORKLOADS[name]
    say(f"[case] full share {name}: generating")
    a = W.generate(w)
    attrs = w.attrs()
    res = run_gpu(a, attrs, torch)
    sel, wts = oracle.route(a["router_probs"], w.k)
    local = oracle.qmoe_oracle.local_experts(sel, w.first_expert, w.held)
    counts, offsets, perm = oracle.expert_permutation(local, w.held + 1)
    check_routing(res, sel, wts, counts[:w.held], offsets[:w.held + 1], perm)
    say(f"  routing bit-exact over {w.tokens} tokens; held-expert slots {counts[:w.held].sum()} of {sel.size}")
    out_all = res["out"].reshape(w.tokens, w.hidden)
    assert np.all(np.isfinite(out_all))
    if w.tokens <= 64:
        ids = list(range(w.tokens))
    else:
        ids = _tile_tokens(counts[:w.held], offsets, perm, w.k)
    say(f"  comparing {len(ids)} of {w.tokens} output rows with the oracle")
    ref = oracle.qmoe_tokens(ids, *a.values(), attrs=attrs)
    check_output(out_all[ids], ref, f"{name} ({len(ids)} rows)")
    # tokens with no slot on the held experts give exact zeros
    none = np.nonzero(~((sel >= w.first_expert) & (sel < w.first_expert + w.held)).any(axis=1))[0]
    assert np.all(out_all[none] == 0.0)
    res2 = run_gpu(a, attrs, torch, debug=False)
    assert np.array_equal(res2["out"], res["out"], equal_nan=False)
