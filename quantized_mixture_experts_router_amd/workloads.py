"""Seeded synthetic QMoE workloads.

This module only draws random inputs; it contains none of the operator's
arithmetic (no routing, no dequantisation, no matmul).  Both the HIP path and
the CPU oracle consume the same host arrays it returns.

Shapes follow the QMoE WebGPU manifest (page "com.microsoft.QMoE manifest",
``inputs``): input (T, H) or (B, S, H) float32; router_probs (T, E) float32;
fc1_experts_weights (E, fusion*I, H/pack) uint8; fc1_scales (E, fusion*I) or
(E, fusion*I, H/bs) float32; fc2_experts_weights (E, H, I/pack) uint8;
fc2_scales (E, H) or (E, H, I/bs) float32, with pack = 2 for 4-bit codes and
fusion = 2 for interleaved SwiGLU.

Draw order (fixed, one ``numpy.random.default_rng(seed)`` per workload):
input ~ N(0, 1); router logits ~ N(0, sigma) (plus the Zipf bias
-2*ln(rank) with rank = e + 1 where requested); fc1 bytes U{0..255};
fc1 scales U[a, b]; fc2 bytes U{0..255}; fc2 scales U[a, b].  Uniform bytes
are uniform 4-bit nibbles as well, so one recipe serves both widths.
"""
from __future__ import annotations

from dataclasses import dataclass, field, asdict
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    input_shape: Tuple[int, ...]   # (T, H) or (B, S, H)
    experts: int
    inter: int
    k: int
    bits: int
    block_size: int                # 0 = column-wise scales
    activation: str                # "relu" | "swiglu"
    scale_range: Tuple[float, float]
    logit_sigma: float = 1.0
    zipf_bias: bool = False
    seed: int = 0
    alpha: float = 1.0
    beta: float = 0.0
    local_experts: int = 0         # > 0: the weights hold this many experts (a share)
    first_expert: int = 0          # global index of the share's first expert

    @property
    def hidden(self) -> int:
        return self.input_shape[-1]

    @property
    def tokens(self) -> int:
        t = 1
        for d in self.input_shape[:-1]:
            t *= d
        return t

    @property
    def held(self) -> int:
        """Experts the weights hold (all of them unless this is a share)."""
        return self.local_experts or self.experts

    @property
    def fusion(self) -> int:
        return 2 if self.activation == "swiglu" else 1

    @property
    def pack(self) -> int:
        return 2 if self.bits == 4 else 1

    def attrs(self) -> dict:
        a = dict(k=self.k, expert_weight_bits=self.bits, block_size=self.block_size,
                 activation_type=self.activation,
                 swiglu_fusion=1 if self.activation == "swiglu" else 0,
                 activation_alpha=self.alpha, activation_beta=self.beta,
                 normalize_routing_weights=0, routing="qmoe")
        if self.local_experts:
            a["first_expert"] = self.first_expert
        return a

    def describe(self) -> dict:
        d = asdict(self)
        d["tokens"] = self.tokens
        return d


# The five measured workloads: a tiny ReLU int8 case, a Mixtral-like int4
# decode step, the same experts at prefill length, a fine-grained 64-expert
# layer with Zipf-skewed routing, and a 128-expert int8 layer.
WORKLOADS = {
    "tiny": Workload("tiny", (8, 64), 4, 128, 1, 8, 0, "relu", (0.005, 0.02)),
    "decode": Workload("decode", (16, 4096), 8, 14336, 2, 4, 64, "swiglu", (0.002, 0.01)),
    "prefill": Workload("prefill", (2, 2048, 4096), 8, 14336, 2, 4, 128, "swiglu", (0.002, 0.01)),
    "fine": Workload("fine", (2048, 2048), 64, 1408, 6, 4, 32, "swiglu", (0.002, 0.01),
                     zipf_bias=True),
    "large_e": Workload("large_e", (4, 2048, 4096), 128, 1536, 8, 8, 0, "swiglu",
                        (0.001, 0.005), logit_sigma=1.5),
}

# One GPU's share of two layers when they are spread over 8 GPUs (the pages
# define no such split; these are the shares measured on one GPU):
#  * large_e_ep8: the 128-expert layer with its experts spread 16 to a GPU;
#    the input and router logits are those of large_e (drawn first, with the
#    same seed, so the routing is large_e's), the weights those of the 16
#    experts from expert 0;
#  * decode_tp8: the decode layer with its inter size split 8 ways (FC1 rows
#    in gate/linear pairs, FC2 columns): inter 14336 / 8 = 1792.
SHARE_WORKLOADS = {
    "large_e_ep8": Workload("large_e_ep8", (4, 2048, 4096), 128, 1536, 8, 8, 0, "swiglu",
                            (0.001, 0.005), logit_sigma=1.5, local_experts=16, first_expert=0),
    "decode_tp8": Workload("decode_tp8", (16, 4096), 8, 1792, 2, 4, 64, "swiglu", (0.002, 0.01)),
}
WORKLOADS.update(SHARE_WORKLOADS)


def shapes(w: Workload) -> dict:
    T, H, E, I = w.tokens, w.hidden, w.experts, w.inter
    F = w.fusion * I
    El = w.held
    d = {
        "input": tuple(w.input_shape),
        "router_probs": (T, E),
        "fc1_experts_weights": (El, F, H // w.pack),
        "fc2_experts_weights": (El, H, I // w.pack),
    }
    if w.block_size:
        d["fc1_scales"] = (El, F, H // w.block_size)
        d["fc2_scales"] = (El, H, I // w.block_size)
    else:
        d["fc1_scales"] = (El, F)
        d["fc2_scales"] = (El, H)
    return d


def generate(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw every input of workload ``w`` in the fixed order documented above."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    s = shapes(w)
    a, b = w.scale_range
    x = rng.standard_normal(s["input"], dtype=np.float32)
    logits = (rng.standard_normal(s["router_probs"], dtype=np.float64) * w.logit_sigma)
    if w.zipf_bias:
        rank = np.arange(1, w.experts + 1, dtype=np.float64)
        logits = logits + (-2.0 * np.log(rank))[None, :]
    logits = logits.astype(np.float32)
    fc1 = rng.integers(0, 256, size=s["fc1_experts_weights"], dtype=np.uint8)
    fc1_s = rng.uniform(a, b, size=s["fc1_scales"]).astype(np.float32)
    fc2 = rng.integers(0, 256, size=s["fc2_experts_weights"], dtype=np.uint8)
    fc2_s = rng.uniform(a, b, size=s["fc2_scales"]).astype(np.float32)
    return {"input": x, "router_probs": logits, "fc1_experts_weights": fc1,
            "fc1_scales": fc1_s, "fc2_experts_weights": fc2, "fc2_scales": fc2_s}


def random_case(rng: np.random.Generator, *, tokens_shape, hidden, experts, inter, k, bits,
                block_size, activation, scale_range=(0.005, 0.02), logit_sigma=1.0) -> tuple:
    """A small random case for sweeps; returns (Workload, arrays)."""
    w = Workload("sweep", tuple(tokens_shape) + (hidden,), experts, inter, k, bits, block_size,
                 activation, scale_range, logit_sigma=logit_sigma)
    return w, generate(w, seed=int(rng.integers(0, 2**31 - 1)))


# ---------------------------------------------------------------- GroupedMatMul
# Float workloads of the standalone GroupedMatMul (ONNX "GroupedMatMul - 29"):
# the FC1 products of the decode and fine-grained layers above with float32
# weights, as a graph that dequantises before the operator would pass them.
# Draw order (one default_rng(seed)): input ~ N(0, 1); weights ~ N(0, 1) *
# wscale; bias ~ N(0, 1) * wscale (when used); group_indices: S distinct
# groups per row, drawn without replacement with probability proportional to
# 1 / rank**2 when zipf is set (the fine-grained layer's skew), else uniform.
@dataclass(frozen=True)
class GmmWorkload:
    name: str
    M: int
    K: int
    G: int
    N: int
    S: int
    bias: bool = True
    zipf: bool = False
    wscale: float = 0.01
    seed: int = 0
    # element type of input, weights, bias and output (the page's Type
    # Constraints): the float32 draws below rounded to it
    dtype: str = "float32"

    def describe(self) -> dict:
        return asdict(self)


GMM_WORKLOADS = {
    "gmm_decode_fc1": GmmWorkload("gmm_decode_fc1", 16, 4096, 8, 28672, 2),
    "gmm_fine_fc1": GmmWorkload("gmm_fine_fc1", 2048, 2048, 64, 2816, 6, zipf=True),
}
# the same two shapes in the page's other element types
for _dt, _sfx in (("float16", "f16"), ("bfloat16", "bf16"), ("float64", "f64")):
    for _base in ("gmm_decode_fc1", "gmm_fine_fc1"):
        _w = GMM_WORKLOADS[_base]
        GMM_WORKLOADS[f"{_base}_{_sfx}"] = GmmWorkload(f"{_base}_{_sfx}", _w.M, _w.K, _w.G, _w.N, _w.S, zipf=_w.zipf,
                                                        dtype=_dt)


def gmm_generate(w: GmmWorkload, seed: Optional[int] = None, index_dtype=np.int64) -> dict:
    """Draw input, weights, group_indices (and bias) of ``w`` in the order above."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    x = rng.standard_normal((w.M, w.K), dtype=np.float32)
    wts = rng.standard_normal((w.G, w.K, w.N), dtype=np.float32)
    wts *= np.float32(w.wscale)
    b = None
    if w.bias:
        b = rng.standard_normal((w.G, w.N), dtype=np.float32) * np.float32(w.wscale)
    p = None
    if w.zipf:
        p = 1.0 / np.arange(1, w.G + 1, dtype=np.float64) ** 2
        p /= p.sum()
    idx = np.empty((w.M, w.S), dtype=index_dtype)
    for m in range(w.M):
        idx[m] = rng.choice(w.G, size=w.S, replace=w.S > w.G, p=p)
    return {"input": x, "weights": wts, "group_indices": idx, "bias": b}


# ---------------------------------------------------------------- float MoE
# Float workloads of the MoE operator (com.microsoft.MoE README): the decode
# and fine-grained layers above with float32 weights and biases.
# Draw order (one default_rng(seed)): input ~ N(0, 1); router logits ~
# N(0, sigma) (plus -2 ln(rank) with rank = e + 1 when zipf is set); fc1
# weights ~ N(0, 1) / sqrt(H); fc1 bias ~ N(0, 1) * 0.1; fc2 weights ~
# N(0, 1) / sqrt(I); fc2 bias ~ N(0, 1) * 0.1; fc3 weights ~ N(0, 1) / sqrt(H);
# fc3 bias ~ N(0, 1) * 0.1 (biases and fc3 only when used).
@dataclass(frozen=True)
class MoeWorkload:
    name: str
    input_shape: Tuple[int, ...]
    experts: int
    inter: int
    k: int
    activation: str = "swiglu"
    fusion: int = 1
    bias: bool = True
    fc3: bool = False
    zipf: bool = False
    logit_sigma: float = 1.0
    normalize: int = 0
    alpha: float = 1.0
    beta: float = 0.0
    seed: int = 0

    @property
    def hidden(self) -> int:
        return self.input_shape[-1]

    @property
    def tokens(self) -> int:
        t = 1
        for d in self.input_shape[:-1]:
            t *= d
        return t

    @property
    def fc1_rows(self) -> int:
        fused = self.activation == "swiglu" and self.fusion in (1, 2)
        return (2 if fused else 1) * self.inter

    def attrs(self) -> dict:
        return dict(k=self.k, activation_type=self.activation, swiglu_fusion=self.fusion,
                    activation_alpha=self.alpha, activation_beta=self.beta,
                    normalize_routing_weights=self.normalize)

    def describe(self) -> dict:
        d = asdict(self)
        d["tokens"] = self.tokens
        return d


MOE_WORKLOADS = {
    "moe_decode": MoeWorkload("moe_decode", (16, 4096), 8, 14336, 2),
    "moe_fine": MoeWorkload("moe_fine", (2048, 2048), 64, 1408, 6, zipf=True),
}


def moe_generate(w: MoeWorkload, seed: Optional[int] = None) -> dict:
    """Draw the inputs of ``w`` in the order above; keys are the operator's
    input names (absent optional inputs are None)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    T, H, E, I, F = w.tokens, w.hidden, w.experts, w.inter, w.fc1_rows

    def normal(shape, scale):
        a = rng.standard_normal(shape, dtype=np.float32)
        a *= np.float32(scale)
        return a

    x = rng.standard_normal(tuple(w.input_shape), dtype=np.float32)
    logits = rng.standard_normal((T, E), dtype=np.float64) * w.logit_sigma
    if w.zipf:
        logits = logits + (-2.0 * np.log(np.arange(1, E + 1, dtype=np.float64)))[None, :]
    logits = logits.astype(np.float32)
    fc1 = normal((E, F, H), 1.0 / np.sqrt(max(H, 1)))
    fc1_b = normal((E, F), 0.1) if w.bias else None
    fc2 = normal((E, H, I), 1.0 / np.sqrt(max(I, 1)))
    fc2_b = normal((E, H), 0.1) if w.bias else None
    fc3 = normal((E, I, H), 1.0 / np.sqrt(max(H, 1))) if w.fc3 else None
    fc3_b = normal((E, I), 0.1) if w.fc3 and w.bias else None
    return {"input": x, "router_probs": logits, "fc1_experts_weights": fc1, "fc1_experts_bias": fc1_b,
            "fc2_experts_weights": fc2, "fc2_experts_bias": fc2_b, "fc3_experts_weights": fc3,
            "fc3_experts_bias": fc3_b}


def moe_random_case(rng: np.random.Generator, *, tokens_shape, hidden, experts, inter, k, activation="relu",
                    fusion=0, bias=True, fc3=False, normalize=0, alpha=1.0, beta=0.0, logit_sigma=1.0) -> tuple:
    """A small random float MoE case for sweeps; returns (MoeWorkload, arrays)."""
    w = MoeWorkload("sweep", tuple(tokens_shape) + (hidden,), experts, inter, k, activation, fusion, bias, fc3,
                    logit_sigma=logit_sigma, normalize=normalize, alpha=alpha, beta=beta)
    return w, moe_generate(w, seed=int(rng.integers(0, 2**31 - 1)))
