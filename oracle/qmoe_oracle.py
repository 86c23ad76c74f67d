"""Plain float64 CPU oracle of the QMoE routed expert FFN — TEST INFRASTRUCTURE.

What the operator computes, step by step, as the pages define it:

* Contract and shapes: QMoE WebGPU manifest, keys ``inputs``, ``outputs``,
  ``attributes``, ``attributeConstraints``, ``typeConstraints`` and the
  ``derive`` expressions ``hiddenSize``, ``numTokens``, ``fusionSize``,
  ``interSize``, ``packSize``, ``quantMidpoint``, ``colWiseScales``,
  ``fc1ScaleBlocks``, ``fc2ScaleBlocks``, ``activationSupported``,
  ``quantBlockSizeOk``, ``quantScalesOk``, ``quantShapeOk``, ``quantContract``.
* Routing: manifest ``description`` (softmax over the selected top-k logits)
  and ``attributeDescriptions.normalize_routing_weights``; the float MoE
  README, section Description (softmax over all logits before top-k, optional
  renormalisation of the selected weights).
* Dequantisation: manifest ``description`` (4- and 8-bit symmetric) with
  ``derive.quantMidpoint`` (8 or 128) and ``derive.packSize`` (2 or 1).
* Expert FFN: FC1, then ReLU or interleaved SwiGLU
  (``attributeDescriptions.swiglu_fusion``, ``activation_alpha``,
  ``activation_beta``), then FC2, each a GroupedMatMul in the sense of the
  ONNX GroupedMatMul-29 page (Summary: weight-only quantised experts are
  DequantizeLinear followed by GroupedMatMul).
* Combine: the routing-weighted sum of the selected experts' outputs (MoE
  README, Description).

Readings taken where the pages are silent:

* low nibble of a packed byte holds the even code index (convention; parity
  unpinned by the pages, pinned only as this convention);
* interleaved SwiGLU: FC1 row 2j is the gate, row 2j+1 the linear branch,
  act = g * sigmoid(alpha * g) * (u + beta);
* the optional swiglu_limit L (``attributeDescriptions.swiglu_limit``; the
  pages give no formula) clamps before that formula: g <- min(g, L),
  u <- clamp(u, -L, L); L must be > 0 (parity unpinned by the pages: pinned
  only by invariants of this reading);
* top-k order is descending logit, equal logits go to the lower expert index,
  and -0.0 equals +0.0;
* the selected-logit softmax subtracts the largest selected logit;
* the expert-sorted slot order is stable (ascending slot id t*k+s);
* a share of the experts (attribute ``first_expert``; the pages define no
  split of the experts): the weights hold E_local consecutive experts from
  global expert ``first_expert``; routing ranks all E logits as always, and
  only slots whose expert is held contribute, so the shares of a partition of
  the experts sum to the whole operator's output.

Everything is float64; inputs are read exactly as stored.
"""
from __future__ import annotations

import numpy as np

ROUTING_QMOE = "qmoe"   # softmax over the k selected logits
ROUTING_MOE = "moe"     # softmax over all logits, then top-k


class ContractError(ValueError):
    """Raised for inputs outside the operator contract.

    ``kind`` is one of "shape", "attr", "unsupported", "dtype".
    """

    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


DEFAULT_ATTRS = dict(activation_alpha=1.0, activation_beta=0.0, activation_type="relu",
                     expert_weight_bits=4, k=1, normalize_routing_weights=0, quant_type="int",
                     swiglu_fusion=0, use_sparse_mixer=0, weights_prepacked=-1, block_size=0,
                     routing=ROUTING_QMOE, swiglu_limit=None, first_expert=0)


def _attrs(attrs: dict | None) -> dict:
    a = dict(DEFAULT_ATTRS)
    if attrs:
        a.update(attrs)
    return a


def validate(x, logits, fc1_w, fc1_s, fc2_w, fc2_s, attrs=None, out_shape=None) -> dict:
    """Check the manifest contract; return the derived sizes.

    Follows the manifest's ``derive`` booleans clause by clause.  Raises
    ContractError on the first violation.
    """
    a = _attrs(attrs)
    # attributeConstraints and the unimplemented standard values
    if a["quant_type"] != "int":
        raise ContractError("unsupported", "quant_type must be int")
    if a["use_sparse_mixer"] not in (0,):
        if a["use_sparse_mixer"] == 1:
            raise ContractError("unsupported", "sparse mixer routing")
        raise ContractError("attr", "use_sparse_mixer")
    if a["weights_prepacked"] not in (-1, 0):
        if a["weights_prepacked"] == 1:
            raise ContractError("unsupported", "provider-prepacked weights")
        raise ContractError("attr", "weights_prepacked")
    if a["swiglu_fusion"] == 2:
        raise ContractError("unsupported", "concatenated SwiGLU fusion")
    if a["expert_weight_bits"] not in (4, 8):
        raise ContractError("attr", "expert_weight_bits must be 4 or 8")
    if a["normalize_routing_weights"] not in (0, 1):
        raise ContractError("attr", "normalize_routing_weights must be 0 or 1")
    if a["routing"] not in (ROUTING_QMOE, ROUTING_MOE):
        raise ContractError("attr", "routing mode")
    act = a["activation_type"]
    fus = a["swiglu_fusion"]
    if not ((act == "relu" and fus == 0) or (act == "swiglu" and fus == 1)):
        raise ContractError("attr", "activation/swiglu_fusion combination")
    bs = int(a["block_size"] or 0)
    if bs < 0 or (bs and (bs < 16 or (bs & (bs - 1)) != 0)):
        raise ContractError("attr", "block_size must be a power of two >= 16")

    # typeConstraints
    for name, arr, dt in (("input", x, np.float32), ("router_probs", logits, np.float32),
                          ("fc1_experts_weights", fc1_w, np.uint8), ("fc1_scales", fc1_s, np.float32),
                          ("fc2_experts_weights", fc2_w, np.uint8), ("fc2_scales", fc2_s, np.float32)):
        if np.asarray(arr).dtype != dt:
            raise ContractError("dtype", f"{name} must be {np.dtype(dt).name}")

    x, logits, fc1_w, fc1_s, fc2_w, fc2_s = (np.asarray(v) for v in (x, logits, fc1_w, fc1_s, fc2_w, fc2_s))
    # inputOutputShapeOk
    if x.ndim not in (2, 3):
        raise ContractError("shape", "input rank must be 2 or 3")
    if out_shape is not None and tuple(out_shape) != tuple(x.shape):
        raise ContractError("shape", "output shape must equal input shape")
    H = x.shape[-1]
    if H <= 0:
        raise ContractError("shape", "hidden size must be positive")
    T = int(np.prod(x.shape[:-1]))
    bits = a["expert_weight_bits"]
    pack = 2 if bits == 4 else 1
    fusion = 2 if (act == "swiglu" and fus == 1) else 1
    # quantShapeOk
    if logits.ndim != 2 or fc1_w.ndim != 3 or fc2_w.ndim != 3:
        raise ContractError("shape", "router rank 2, weights rank 3")
    E = logits.shape[1]
    if logits.shape[0] != T:
        raise ContractError("shape", "router rows must equal the token count")
    El = fc1_w.shape[0]  # experts the weights hold (a share: fewer than E)
    if El > E or fc2_w.shape[0] != El:
        raise ContractError("shape", "expert count mismatch")
    first = int(a["first_expert"])
    if first < 0 or first + El > E:
        raise ContractError("attr", "first_expert + held experts must lie in [0, num_experts]")
    F = fc1_w.shape[1]
    if F % fusion != 0:
        raise ContractError("shape", "fc1 rows not divisible by the fusion size")
    I = F // fusion
    if fc2_w.shape[1] != H:
        raise ContractError("shape", "fc2 rows must equal hidden size")
    if fc1_w.shape[2] * pack != H or fc2_w.shape[2] * pack != I:
        raise ContractError("shape", "packed column count mismatch")
    if bs and (H % bs != 0 or I % bs != 0):
        raise ContractError("shape", "block_size must divide hidden and inter size")
    # quantScalesOk
    if fc1_s.shape[:2] != (El, F) or fc2_s.shape[:2] != (El, H):
        raise ContractError("shape", "scale leading dims")
    if bs == 0:
        if fc1_s.ndim != 2 or fc2_s.ndim != 2:
            raise ContractError("shape", "column-wise scales must be rank 2")
    else:
        if fc1_s.ndim != 3 or fc2_s.ndim != 3 or fc1_s.shape[2] != H // bs or fc2_s.shape[2] != I // bs:
            raise ContractError("shape", "blockwise scales must be rank 3 with H/bs and I/bs blocks")
    # quantContract: 1 <= k <= E
    k = a["k"]
    if not (1 <= k <= E):
        raise ContractError("attr", "k must lie in [1, num_experts]")
    limit = swiglu_limit_of(a)
    return dict(T=T, H=H, E=E, El=El, first=first, I=I, F=F, k=k, bits=bits, pack=pack, fusion=fusion, bs=bs,
                mid=8 if bits == 4 else 128, activation=act, alpha=float(a["activation_alpha"]),
                beta=float(a["activation_beta"]), routing=a["routing"],
                normalize=int(a["normalize_routing_weights"]), limit=limit)


def route(logits, k: int, routing: str = ROUTING_QMOE, normalize: int = 0):
    """Top-k selection and routing weights for every token.

    Selection: the k largest float32 logits of a row, largest first, equal
    values ordered by ascending expert index (lexsort on (index, -logit)).
    QMoE weights: softmax over the selected logits (manifest ``description``).
    MoE weights: softmax over all logits, taken at the selection, divided by
    their sum when ``normalize`` is 1 (MoE README, Description).
    """
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -L), axis=-1)      # last key is primary
    sel = order[:, :k].astype(np.int64)
    Ls = np.take_along_axis(L, sel, axis=1).astype(np.float64)
    if routing == ROUTING_QMOE:
        e = np.exp(Ls - Ls[:, :1])
        w = e / e.sum(axis=1, keepdims=True)
    else:
        L64 = L.astype(np.float64)
        p = np.exp(L64 - L64.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, sel, axis=1)
        if normalize:
            w = w / w.sum(axis=1, keepdims=True)
    return sel, w


def expert_permutation(sel, num_experts: int):
    """Per-expert counts, exclusive offsets and the stable expert-sorted order.

    ``perm[p]`` is the slot id t*k+s at sorted position p; slots of one
    expert appear in ascending slot id (a stable sort by expert).
    """
    flat = np.asarray(sel).reshape(-1)
    counts = np.bincount(flat, minlength=num_experts).astype(np.int64)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    return counts, offsets, perm


def local_experts(sel, first: int, held: int):
    """Index of each selected expert among the held ones [first, first +
    held), or ``held`` for an expert not held."""
    sel = np.asarray(sel)
    inside = (sel >= first) & (sel < first + held)
    return np.where(inside, sel - first, held)


def unpack_codes(packed, bits: int):
    """Integer codes from raw packed bytes; 4-bit: low nibble is the even code."""
    b = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return b.astype(np.int64)
    lo = (b & 0x0F).astype(np.int64)
    hi = (b >> 4).astype(np.int64)
    q = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    return q


def dequantize(packed, scales, bits: int, block_size: int):
    """W = (q - midpoint) * scale, exactly, in float64.

    Midpoint 8 (4-bit) or 128 (8-bit).  Column-wise scales are one per output
    row; blockwise scales hold one value per ``block_size`` reduction columns.
    Works on one expert ([N, K/pack]) or a stack ([E, N, K/pack]).
    """
    q = unpack_codes(packed, bits)
    mid = 8 if bits == 4 else 128
    s = np.asarray(scales, dtype=np.float64)
    if block_size == 0:
        S = s[..., None]
    else:
        S = np.repeat(s, block_size, axis=-1)
    return (q - mid).astype(np.float64) * S


def swiglu_limit_of(a: dict) -> float:
    """The optional SwiGLU clamp limit (QMoE manifest
    ``attributeDescriptions.swiglu_limit``, ``constants.hasSwigluLimit``):
    +inf when absent; a present limit must be a number > 0."""
    v = a.get("swiglu_limit")
    if v is None:
        return float("inf")
    v = float(v)
    if not v > 0:
        raise ContractError("attr", "swiglu_limit must be > 0")
    return v


def clamp_swiglu(g, u, limit: float):
    """Reading of the clamp (the pages give no formula): the gate is bounded
    above by the limit, the linear branch on both sides."""
    return np.minimum(g, limit), np.clip(u, -limit, limit)


def activation(h, act: str, alpha: float = 1.0, beta: float = 0.0, limit: float = float("inf")):
    """ReLU, or interleaved SwiGLU over FC1 row pairs (gate 2j, linear 2j+1),
    with the optional clamp limit."""
    h = np.asarray(h, dtype=np.float64)
    if act == "relu":
        return np.maximum(h, 0.0)
    g, u = clamp_swiglu(h[..., 0::2], h[..., 1::2], limit)
    return g / (1.0 + np.exp(-alpha * g)) * (u + beta)


def expert_ffn(xrows, w1, w2, act, alpha, beta, limit=float("inf")):
    """FC1 -> activation -> FC2 for the rows routed to one expert (float64)."""
    h = np.asarray(xrows, dtype=np.float64) @ w1.T
    a = activation(h, act, alpha, beta, limit)
    return a @ w2.T


def qmoe(x, logits, fc1_w, fc1_s, fc2_w, fc2_s, attrs=None, return_intermediates=False):
    """The routed operator: route, group slots by expert, run each expert once
    over its rows, then take the routing-weighted sum per token.

    Returns the float64 output in the input's shape (callers cast to float32
    where they need the operator's output type).
    """
    d = validate(x, logits, fc1_w, fc1_s, fc2_w, fc2_s, attrs)
    T, H, El, I, k = d["T"], d["H"], d["El"], d["I"], d["k"]
    xs = np.asarray(x, dtype=np.float32).reshape(T, H).astype(np.float64)
    sel, w = route(logits, k, d["routing"], d["normalize"])
    # slots grouped by held expert; the slots of experts not held form one
    # more group after them (they contribute nothing)
    local = local_experts(sel, d["first"], El)
    counts, offsets, perm = expert_permutation(local, El + 1)
    slot_out = np.zeros((T * k, H), dtype=np.float64)
    if I > 0:
        for e in range(El):
            if counts[e] == 0:
                continue
            rows = perm[offsets[e]:offsets[e + 1]]
            w1 = dequantize(fc1_w[e], fc1_s[e], d["bits"], d["bs"])
            w2 = dequantize(fc2_w[e], fc2_s[e], d["bits"], d["bs"])
            slot_out[rows] = expert_ffn(xs[rows // k], w1, w2, d["activation"], d["alpha"], d["beta"], d["limit"])
    out = (w.reshape(T, k, 1) * slot_out.reshape(T, k, H)).sum(axis=1)
    out = out.reshape(np.asarray(x).shape)
    if return_intermediates:
        return out, dict(sel=sel, w=w, counts=counts[:El], offsets=offsets[:El + 1], perm=perm, slot_out=slot_out)
    return out


def qmoe_tokens(token_ids, x, logits, fc1_w, fc1_s, fc2_w, fc2_s, attrs=None):
    """The operator's output rows for a subset of tokens only (float64 [n, H]).

    A token's output depends only on its own input row and logits row, so a
    sample of rows can be checked at full problem size.
    """
    d = validate(x, logits, fc1_w, fc1_s, fc2_w, fc2_s, attrs)
    T, H, k = d["T"], d["H"], d["k"]
    ids = np.asarray(token_ids, dtype=np.int64)
    xs = np.asarray(x, dtype=np.float32).reshape(T, H)[ids].astype(np.float64)
    sel, w = route(np.asarray(logits)[ids], k, d["routing"], d["normalize"])
    out = np.zeros((len(ids), H), dtype=np.float64)
    if d["I"] == 0:
        return out
    local = local_experts(sel, d["first"], d["El"])
    for e in np.unique(local):
        if e == d["El"]:
            continue  # expert not held
        hit = np.nonzero(local == e)
        rows = hit[0]
        w1 = dequantize(fc1_w[e], fc1_s[e], d["bits"], d["bs"])
        w2 = dequantize(fc2_w[e], fc2_s[e], d["bits"], d["bs"])
        y = expert_ffn(xs[rows], w1, w2, d["activation"], d["alpha"], d["beta"], d["limit"])
        for r, (t, s) in enumerate(zip(*hit)):
            out[t] += w[t, s] * y[r]
    return out


def qmoe_dense(x, logits, fc1_w, fc1_s, fc2_w, fc2_s, attrs=None):
    """Brute force, for tiny inputs: dequantise every expert, run every token
    through every expert, then out[t] = sum_s w[t,s] * FFN_{sel[t,s]}(x[t]).

    This is the GroupedMatMul decomposition (gather, expand, matmul) applied to
    dequantised weights, with no grouping or permutation.
    """
    d = validate(x, logits, fc1_w, fc1_s, fc2_w, fc2_s, attrs)
    T, H, E, k = d["T"], d["H"], d["E"], d["k"]
    xs = np.asarray(x, dtype=np.float32).reshape(T, H).astype(np.float64)
    sel, w = route(logits, k, d["routing"], d["normalize"])
    W1 = dequantize(fc1_w, fc1_s, d["bits"], d["bs"])
    W2 = dequantize(fc2_w, fc2_s, d["bits"], d["bs"])
    out = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for s in range(k):
            e = int(sel[t, s]) - d["first"]
            if d["I"] == 0 or not 0 <= e < d["El"]:
                continue
            h = np.zeros(d["F"])
            for n in range(d["F"]):
                h[n] = float(np.dot(W1[e, n], xs[t]))
            a = activation(h, d["activation"], d["alpha"], d["beta"], d["limit"])
            y = np.array([float(np.dot(W2[e, c], a)) for c in range(H)])
            out[t] += w[t, s] * y
    return out.reshape(np.asarray(x).shape)
