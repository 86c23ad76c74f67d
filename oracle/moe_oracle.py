"""Float MoE operator, written out from its page (com.microsoft.MoE README:
Description, Inputs, Outputs, Attributes) in float64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the operator computes, per token t with input row x:
  p        = softmax over all E router logits of t
  sel      = the k experts with the largest logits (ties: lower index first)
  w[s]     = p[sel[s]], divided by sum_s p[sel[s]] when
             normalize_routing_weights = 1
  h        = W1[e] x + b1[e]               (FC1, rows = fusion_size * I)
  a        = activation(h [, FC3 u3 = W3[e] x + b3[e]])
  y        = W2[e] a + b2[e]               (FC2; its bias before the weight)
  out[t]   = sum_s w[s] * y(sel[s])

Readings where the page states no formula (each is listed, with its pin, in
the design notes; parity beyond these readings is unpinned by the pages):
  * weights project by rows: fc1 (E, fusion*I, H), fc2 (E, H, I), fc3
    (E, I, H), as the input table's shapes imply;
  * gelu is the exact form h Phi(h) = 0.5 h (1 + erf(h / sqrt 2));
  * silu is h * sigmoid(h); when FC3 is present it multiplies the result
    (the page's "multiplicative linear projection"); alpha and beta are not
    read by silu, gelu, relu or identity;
  * swiglu is g * sigmoid(alpha g) * (u + beta), the formula the QMoE manifest
    fixes for its SwiGLU attributes, with gate/linear operands
      fusion 0: g = FC1 output, u = FC3 output;
      fusion 1: g = h[2j], u = h[2j+1]  (interleaved, as in QMoE);
      fusion 2: g = h[j],  u = h[I + j] (concatenated, gate block first);
  * fusion_size is 2 only for swiglu with fusion 1 or 2; the swiglu_fusion
    attribute is not read by other activations;
  * FC3 is read only by swiglu with fusion 0 (required there) and by silu
    (optional); other activations ignore it;
  * the optional swiglu_limit L (README Attributes: a SwiGLU clamp, none when
    omitted) bounds the gate above by L and the linear branch to [-L, L]
    before the formula; it must be > 0 and only swiglu reads it.
"""
from __future__ import annotations

import math

import numpy as np

from .qmoe_oracle import ContractError, ROUTING_MOE, clamp_swiglu, expert_permutation, route, swiglu_limit_of

ACTIVATIONS = ("relu", "gelu", "silu", "swiglu", "identity")

DEFAULTS = dict(k=1, activation_type="relu", swiglu_fusion=0, activation_alpha=1.0, activation_beta=0.0,
                normalize_routing_weights=0, use_sparse_mixer=0, swiglu_limit=None)


def moe_attrs(attrs: dict | None) -> dict:
    """Page defaults (Attributes table) overridden by ``attrs``."""
    a = dict(DEFAULTS)
    a.update(attrs or {})
    return a


def _shape(t):
    return None if t is None else tuple(np.shape(t))


def moe_validate(x, logits, fc1_w, fc2_w, fc3_w=None, fc1_b=None, fc2_b=None, fc3_b=None, attrs=None):
    """Sizes of the call, or ContractError(kind) with kind in shape / attr /
    unsupported (Inputs and Attributes tables)."""
    a = moe_attrs(attrs)
    xs = _shape(x)
    if xs is None or len(xs) not in (2, 3):
        raise ContractError("shape", "input must be rank 2 or 3")
    H = xs[-1]
    T = int(np.prod(xs[:-1]))
    ls = _shape(logits)
    if ls is None or len(ls) != 2 or ls[0] != T:
        raise ContractError("shape", "router_probs must be (num_tokens, num_experts)")
    E = ls[1]
    w2 = _shape(fc2_w)
    if w2 is None or len(w2) != 3 or w2[0] != E or w2[1] != H:
        raise ContractError("shape", "fc2_experts_weights must be (E, H, I)")
    I = w2[2]
    act = a["activation_type"]
    if act not in ACTIVATIONS:
        raise ContractError("attr", f"activation_type {act!r}")
    fusion = int(a["swiglu_fusion"])
    if fusion not in (0, 1, 2):
        raise ContractError("attr", "swiglu_fusion must be 0, 1 or 2")
    if int(a["use_sparse_mixer"]) not in (0, 1):
        raise ContractError("attr", "use_sparse_mixer must be 0 or 1")
    if int(a["use_sparse_mixer"]) == 1:
        raise ContractError("unsupported", "sparse mixing is not implemented")
    if int(a["normalize_routing_weights"]) not in (0, 1):
        raise ContractError("attr", "normalize_routing_weights must be 0 or 1")
    k = int(a["k"])
    if k < 1 or k > E:
        raise ContractError("attr", "k must satisfy 1 <= k <= num_experts")
    fused = act == "swiglu" and fusion in (1, 2)
    F = (2 if fused else 1) * I
    if _shape(fc1_w) != (E, F, H):
        raise ContractError("shape", f"fc1_experts_weights must be {(E, F, H)}")
    if fc3_w is not None and _shape(fc3_w) != (E, I, H):
        raise ContractError("shape", f"fc3_experts_weights must be {(E, I, H)}")
    if act == "swiglu" and fusion == 0 and fc3_w is None:
        raise ContractError("shape", "swiglu with swiglu_fusion 0 needs fc3_experts_weights")
    if fc1_b is not None and _shape(fc1_b) != (E, F):
        raise ContractError("shape", "fc1_experts_bias must be (E, fusion_size * I)")
    if fc2_b is not None and _shape(fc2_b) != (E, H):
        raise ContractError("shape", "fc2_experts_bias must be (E, H)")
    if fc3_b is not None and (fc3_w is None or _shape(fc3_b) != (E, I)):
        raise ContractError("shape", "fc3_experts_bias must be (E, I) and come with fc3 weights")
    uses_fc3 = fc3_w is not None and (act == "silu" or (act == "swiglu" and fusion == 0))
    limit = swiglu_limit_of(a)
    return dict(T=T, H=H, E=E, I=I, F=F, k=k, act=act, fusion=fusion, fused=fused, uses_fc3=uses_fc3,
                alpha=float(a["activation_alpha"]), beta=float(a["activation_beta"]),
                normalize=int(a["normalize_routing_weights"]), limit=limit)


def gelu(h):
    """Exact GELU: h * Phi(h), Phi the standard normal CDF, written as
    erfc(-h / sqrt 2) / 2 (equal to (1 + erf(h / sqrt 2)) / 2 without its
    cancellation for negative h)."""
    h = np.asarray(h, dtype=np.float64)
    erfc = np.vectorize(math.erfc, otypes=[np.float64])
    return 0.5 * h * erfc(-h / math.sqrt(2.0))


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-np.asarray(v, dtype=np.float64)))


def moe_activation(h, act, fusion=0, alpha=1.0, beta=0.0, u3=None, limit=float("inf")):
    """Activation of one FC1 output vector h (and the FC3 output u3 when read)."""
    h = np.asarray(h, dtype=np.float64)
    if act == "relu":
        return np.maximum(h, 0.0)
    if act == "identity":
        return h.copy()
    if act == "gelu":
        return gelu(h)
    if act == "silu":
        s = h * sigmoid(h)
        return s * u3 if u3 is not None else s
    # swiglu
    if fusion == 0:
        g, u = h, u3
    elif fusion == 1:
        g, u = h[..., 0::2], h[..., 1::2]
    else:
        half = h.shape[-1] // 2
        g, u = h[..., :half], h[..., half:]
    g, u = clamp_swiglu(g, u, limit)
    return g * sigmoid(alpha * g) * (u + beta)


def moe_expert(xrow, e, d, fc1_w, fc2_w, fc3_w=None, fc1_b=None, fc2_b=None, fc3_b=None):
    """y = FC2(activation(FC1 x [, FC3 x])) of expert e for one token row (float64)."""
    x = np.asarray(xrow, dtype=np.float64)
    h = np.asarray(fc1_w[e], dtype=np.float64) @ x
    if fc1_b is not None:
        h = h + np.asarray(fc1_b[e], dtype=np.float64)
    u3 = None
    if d["uses_fc3"]:
        u3 = np.asarray(fc3_w[e], dtype=np.float64) @ x
        if fc3_b is not None:
            u3 = u3 + np.asarray(fc3_b[e], dtype=np.float64)
    a = moe_activation(h, d["act"], d["fusion"], d["alpha"], d["beta"], u3, d["limit"])
    y = np.asarray(fc2_w[e], dtype=np.float64) @ a
    if fc2_b is not None:
        y = y + np.asarray(fc2_b[e], dtype=np.float64)
    return y


def moe_tokens(token_ids, x, logits, fc1_w, fc2_w, fc3_w=None, fc1_b=None, fc2_b=None, fc3_b=None, attrs=None,
               return_routing=False):
    """Output rows (float64) of the listed tokens, each computed on its own."""
    d = moe_validate(x, logits, fc1_w, fc2_w, fc3_w, fc1_b, fc2_b, fc3_b, attrs)
    T, H = d["T"], d["H"]
    xs = np.asarray(x, dtype=np.float32).reshape(T, H)
    L = np.asarray(logits, dtype=np.float32)
    ids = list(token_ids)
    out = np.zeros((len(ids), H), dtype=np.float64)
    sels, ws = [], []
    for r, t in enumerate(ids):
        sel, w = route(L[t:t + 1], d["k"], ROUTING_MOE, d["normalize"])
        for s in range(d["k"]):
            out[r] += w[0, s] * moe_expert(xs[t], int(sel[0, s]), d, fc1_w, fc2_w, fc3_w, fc1_b, fc2_b, fc3_b)
        sels.append(sel[0])
        ws.append(w[0])
    if return_routing:
        return out, np.array(sels).reshape(len(ids), d["k"]), np.array(ws).reshape(len(ids), d["k"])
    return out


def moe(x, logits, fc1_w, fc2_w, fc3_w=None, fc1_b=None, fc2_b=None, fc3_b=None, attrs=None,
        return_intermediates=False):
    """The whole operator: float64 output in the input's shape."""
    d = moe_validate(x, logits, fc1_w, fc2_w, fc3_w, fc1_b, fc2_b, fc3_b, attrs)
    T = d["T"]
    out, sel, w = moe_tokens(range(T), x, logits, fc1_w, fc2_w, fc3_w, fc1_b, fc2_b, fc3_b, attrs,
                             return_routing=True)
    out = out.reshape(np.shape(x))
    if not return_intermediates:
        return out
    sel = sel.reshape(T, d["k"]).astype(np.int64)
    counts, offsets, perm = expert_permutation(sel, d["E"])
    return out, dict(sel=sel, w=w.reshape(T, d["k"]), counts=counts, offsets=offsets, perm=perm, dims=d)
