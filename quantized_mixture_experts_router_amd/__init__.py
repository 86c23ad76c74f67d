"""Python binding of libqmoe.so, the QMoE routed expert FFN for gfx950.

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the C ABI of include/qmoe.h.  PyTorch supplies device memory
and the current stream.  The functions keep the C names:

    qmoe_abi_version, qmoe_attrs_default, qmoe_validate, qmoe_workspace_size,
    qmoe_plan_describe, qmoe_forward, qmoe_forward_debug, qmoe_forward_noalloc,
    qmoe_noalloc_scratch_bytes, qmoe_status_string,
    qmoe_grouped_matmul_workspace_size, qmoe_grouped_matmul,
    qmoe_grouped_matmul_debug, qmoe_moe_attrs_default, qmoe_moe_validate,
    qmoe_moe_workspace_size, qmoe_moe_forward, qmoe_moe_forward_debug

plus ``forward``, ``grouped_matmul`` and ``moe_forward`` (allocate output and
workspace with torch, then call the entry point) for convenience.  The
library is loaded on first use; a missing build raises immediately, there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")

QMOE_F32, QMOE_U8, QMOE_I32, QMOE_I64, QMOE_F16, QMOE_BF16, QMOE_F64 = 1, 2, 3, 4, 5, 6, 7
QMOE_ACT = {"relu": 0, "swiglu": 1, "gelu": 2, "silu": 3, "identity": 4}
QMOE_ROUTING = {"qmoe": 0, "moe": 1}
STATUS = {0: "OK", 1: "NULL", 2: "SHAPE", 3: "ATTR", 4: "UNSUPPORTED", 5: "WORKSPACE", 6: "HIP",
          7: "DTYPE", 8: "ALIGN"}


class QmoeTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("dims", ctypes.c_int64 * 3)]


class QmoeAttrs(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("expert_weight_bits", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("activation_type", ctypes.c_int32), ("swiglu_fusion", ctypes.c_int32),
                ("activation_alpha", ctypes.c_float), ("activation_beta", ctypes.c_float),
                ("normalize_routing_weights", ctypes.c_int32), ("routing", ctypes.c_int32),
                ("use_sparse_mixer", ctypes.c_int32), ("weights_prepacked", ctypes.c_int32),
                ("quant_type", ctypes.c_int32), ("has_swiglu_limit", ctypes.c_int32),
                ("swiglu_limit", ctypes.c_float), ("first_expert", ctypes.c_int32)]


class QmoeMoeAttrs(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("activation_type", ctypes.c_int32), ("swiglu_fusion", ctypes.c_int32),
                ("activation_alpha", ctypes.c_float), ("activation_beta", ctypes.c_float),
                ("normalize_routing_weights", ctypes.c_int32), ("use_sparse_mixer", ctypes.c_int32),
                ("has_swiglu_limit", ctypes.c_int32), ("swiglu_limit", ctypes.c_float)]


QMOE_STAGE_EVENTS = 6
QMOE_GMM_EVENTS = 3


class QmoeDebug(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("events", ctypes.c_void_p * QMOE_STAGE_EVENTS)]


class QmoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({qmoe_status_string(status)})")
        self.status = status
        self.name = STATUS.get(status, str(status))


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m quantized_mixture_experts_router_amd.build`")
        # torch ships its own HIP runtime under the same soname; loading torch
        # first makes this library bind to that one copy (one runtime per process).
        import torch  # noqa: F401
        lib = ctypes.CDLL(LIB_PATH)
        T = ctypes.POINTER(QmoeTensor)
        A = ctypes.POINTER(QmoeAttrs)
        lib.qmoe_abi_version.restype = ctypes.c_int32
        lib.qmoe_attrs_default.argtypes = [A]
        lib.qmoe_attrs_default.restype = None
        lib.qmoe_validate.argtypes = [T, T, T, T, T, T, T, A]
        lib.qmoe_validate.restype = ctypes.c_int
        lib.qmoe_workspace_size.argtypes = [T, T, T, T, T, T, A, ctypes.POINTER(ctypes.c_size_t)]
        lib.qmoe_workspace_size.restype = ctypes.c_int
        lib.qmoe_forward.argtypes = [T, T, T, T, T, T, A, T, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.qmoe_forward.restype = ctypes.c_int
        lib.qmoe_forward_debug.argtypes = [T, T, T, T, T, T, A, T, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p, ctypes.POINTER(QmoeDebug)]
        lib.qmoe_forward_debug.restype = ctypes.c_int
        lib.qmoe_plan_describe.argtypes = [T, T, T, T, T, T, A, ctypes.c_char_p, ctypes.c_size_t]
        lib.qmoe_plan_describe.restype = ctypes.c_int
        lib.qmoe_noalloc_scratch_bytes.argtypes = []
        lib.qmoe_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.qmoe_forward_noalloc.argtypes = [T, T, T, T, T, T, A, T, ctypes.c_void_p]
        lib.qmoe_forward_noalloc.restype = ctypes.c_int
        lib.qmoe_grouped_matmul_workspace_size.argtypes = [T, T, T, T, T, ctypes.POINTER(ctypes.c_size_t)]
        lib.qmoe_grouped_matmul_workspace_size.restype = ctypes.c_int
        lib.qmoe_grouped_matmul.argtypes = [T, T, T, T, T, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.qmoe_grouped_matmul.restype = ctypes.c_int
        lib.qmoe_grouped_matmul_debug.argtypes = [T, T, T, T, T, ctypes.c_void_p, ctypes.c_size_t,
                                                  ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
        lib.qmoe_grouped_matmul_debug.restype = ctypes.c_int
        MA = ctypes.POINTER(QmoeMoeAttrs)
        lib.qmoe_moe_attrs_default.argtypes = [MA]
        lib.qmoe_moe_attrs_default.restype = None
        lib.qmoe_moe_validate.argtypes = [T] * 9 + [MA]
        lib.qmoe_moe_validate.restype = ctypes.c_int
        lib.qmoe_moe_workspace_size.argtypes = [T] * 8 + [MA, ctypes.POINTER(ctypes.c_size_t)]
        lib.qmoe_moe_workspace_size.restype = ctypes.c_int
        lib.qmoe_moe_forward.argtypes = [T] * 8 + [MA, T, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.qmoe_moe_forward.restype = ctypes.c_int
        lib.qmoe_moe_forward_debug.argtypes = [T] * 8 + [MA, T, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                         ctypes.POINTER(QmoeDebug)]
        lib.qmoe_moe_forward_debug.restype = ctypes.c_int
        lib.qmoe_status_string.argtypes = [ctypes.c_int]
        lib.qmoe_status_string.restype = ctypes.c_char_p
        _lib_handle = lib
    return _lib_handle


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


# ------------------------------------------------------------------ marshalling
def describe(t, data: bool = True) -> QmoeTensor:
    """qmoe_tensor for a torch tensor or numpy array (shape, dtype, pointer)."""
    shape = tuple(t.shape)  # ranks above 3 pass through so the library rejects them
    name = str(t.dtype).replace("torch.", "")
    code = {"float32": QMOE_F32, "uint8": QMOE_U8, "int32": QMOE_I32, "int64": QMOE_I64, "float16": QMOE_F16,
            "bfloat16": QMOE_BF16, "float64": QMOE_F64}.get(name, 0)
    ptr = None
    if data and hasattr(t, "data_ptr"):
        if not t.is_contiguous():
            raise ValueError("qmoe tensors must be contiguous")
        ptr = t.data_ptr() if t.numel() > 0 else None
    d = QmoeTensor()
    d.data = ptr
    d.dtype = code
    d.rank = len(shape)
    for i in range(3):
        d.dims[i] = shape[i] if i < len(shape) else 0
    return d


def make_attrs(attrs: Optional[dict] = None) -> QmoeAttrs:
    a = qmoe_attrs_default()
    for key, val in (attrs or {}).items():
        if key == "activation_type":
            val = QMOE_ACT.get(val, 99) if isinstance(val, str) else val
        elif key == "routing":
            val = QMOE_ROUTING.get(val, 99) if isinstance(val, str) else val
        elif key == "quant_type":
            val = 0 if val in ("int", 0) else 1
        elif key == "block_size" and val is None:
            val = 0
        elif key == "swiglu_limit":
            # absent (None) or a value; a given value is passed as is and
            # the library checks it
            a.has_swiglu_limit = 0 if val is None else 1
            val = 0.0 if val is None else val
        setattr(a, key, val)
    return a


# ------------------------------------------------------------------ C entry points
def qmoe_abi_version() -> int:
    return int(_lib().qmoe_abi_version())


def qmoe_status_string(status: int) -> str:
    return _lib().qmoe_status_string(int(status)).decode()


def qmoe_attrs_default() -> QmoeAttrs:
    a = QmoeAttrs()
    _lib().qmoe_attrs_default(ctypes.byref(a))
    return a


def _six(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, data=True):
    return [describe(t, data) for t in (input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s)]


def qmoe_validate(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, output=None, attrs=None) -> int:
    """Status code of the contract check (0 = OK).  Arrays may live anywhere."""
    ts = _six(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, data=False)
    out = ctypes.byref(describe(output, False)) if output is not None else None
    a = attrs if isinstance(attrs, QmoeAttrs) else make_attrs(attrs)
    return int(_lib().qmoe_validate(*[ctypes.byref(t) for t in ts], out, ctypes.byref(a)))


def qmoe_workspace_size(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, attrs=None) -> int:
    ts = _six(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, data=False)
    a = attrs if isinstance(attrs, QmoeAttrs) else make_attrs(attrs)
    n = ctypes.c_size_t(0)
    st = _lib().qmoe_workspace_size(*[ctypes.byref(t) for t in ts], ctypes.byref(a), ctypes.byref(n))
    if st != 0:
        raise QmoeError(st, "qmoe_workspace_size")
    return int(n.value)


def qmoe_plan_describe(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, attrs=None) -> str:
    """The launch plan of qmoe_forward for these shapes, as one line of text.
    Arrays may live anywhere (only shapes and dtypes are read)."""
    ts = _six(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, data=False)
    a = attrs if isinstance(attrs, QmoeAttrs) else make_attrs(attrs)
    buf = ctypes.create_string_buffer(512)
    st = _lib().qmoe_plan_describe(*[ctypes.byref(t) for t in ts], ctypes.byref(a), buf, 512)
    if st != 0:
        raise QmoeError(st, "qmoe_plan_describe")
    return buf.value.decode()


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def qmoe_forward(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, attrs, output, workspace, stream=None,
                 debug: Optional[dict] = None) -> None:
    """Enqueue the operator on ``stream`` (default: torch's current stream).

    All tensors are contiguous device tensors; ``workspace`` is a uint8 device
    tensor of at least qmoe_workspace_size bytes (or None when that size is 0).
    ``debug`` may map topk_idx / topk_w / counts / offsets / perm to device
    tensors that receive the routing stages' results, and ``events`` to up to
    QMOE_STAGE_EVENTS raw hipEvent_t handles (qmoe_forward_debug).
    """
    ts = _six(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s)
    o = describe(output)
    a = attrs if isinstance(attrs, QmoeAttrs) else make_attrs(attrs)
    wptr = workspace.data_ptr() if workspace is not None and workspace.numel() > 0 else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = [*[ctypes.byref(t) for t in ts], ctypes.byref(a), ctypes.byref(o), ctypes.c_void_p(wptr),
            ctypes.c_size_t(wbytes), _stream_handle(stream)]
    if debug is None:
        st = _lib().qmoe_forward(*args)
        where = "qmoe_forward"
    else:
        dbg = QmoeDebug()
        for f in ("topk_idx", "topk_w", "counts", "offsets", "perm"):
            t = debug.get(f)
            setattr(dbg, f, t.data_ptr() if t is not None and t.numel() > 0 else None)
        for i, ev in enumerate(debug.get("events") or ()):
            dbg.events[i] = ev  # raw hipEvent_t handles
        st = _lib().qmoe_forward_debug(*args, ctypes.byref(dbg))
        where = "qmoe_forward_debug"
    if st != 0:
        raise QmoeError(st, where)


qmoe_forward_debug = qmoe_forward


def qmoe_noalloc_scratch_bytes() -> int:
    """Size of the library's per-GPU scratch array used by qmoe_forward_noalloc."""
    return int(_lib().qmoe_noalloc_scratch_bytes())


def qmoe_forward_noalloc(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, attrs, output, stream=None) -> None:
    """qmoe_forward without a workspace: the library's per-GPU scratch array
    holds the intermediates (calls on one GPU must not overlap)."""
    ts = _six(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s)
    o = describe(output)
    a = attrs if isinstance(attrs, QmoeAttrs) else make_attrs(attrs)
    st = _lib().qmoe_forward_noalloc(*[ctypes.byref(t) for t in ts], ctypes.byref(a), ctypes.byref(o),
                                     _stream_handle(stream))
    if st != 0:
        raise QmoeError(st, "qmoe_forward_noalloc")


def forward(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, attrs=None, stream=None, workspace=None,
            output=None, debug=None):
    """Allocate output (and workspace unless given) with torch, then qmoe_forward."""
    import torch
    if output is None:
        output = torch.empty_like(input)
    need = qmoe_workspace_size(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, attrs)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=input.device)
    qmoe_forward(input, router_probs, fc1_w, fc1_s, fc2_w, fc2_s, attrs, output, workspace, stream, debug)
    return output


def _ref(t, data):
    return ctypes.byref(describe(t, data)) if t is not None else None


def qmoe_grouped_matmul_workspace_size(input, weights, group_indices, bias=None, output=None) -> int:
    """Workspace bytes of qmoe_grouped_matmul.  Arrays may live anywhere."""
    n = ctypes.c_size_t(0)
    st = _lib().qmoe_grouped_matmul_workspace_size(_ref(input, False), _ref(weights, False),
                                                   _ref(group_indices, False), _ref(bias, False),
                                                   _ref(output, False), ctypes.byref(n))
    if st != 0:
        raise QmoeError(st, "qmoe_grouped_matmul_workspace_size")
    return int(n.value)


def qmoe_grouped_matmul(input, weights, group_indices, bias, output, workspace, stream=None, events=None) -> None:
    """Enqueue GroupedMatMul on ``stream`` (default: torch's current stream).

    Contiguous device tensors; ``bias`` may be None; ``workspace`` a uint8
    device tensor of at least qmoe_grouped_matmul_workspace_size bytes (or
    None when that size is 0).  ``events``: up to QMOE_GMM_EVENTS raw
    hipEvent_t handles (calls qmoe_grouped_matmul_debug).
    """
    wptr = workspace.data_ptr() if workspace is not None and workspace.numel() > 0 else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = [_ref(input, True), _ref(weights, True), _ref(group_indices, True), _ref(bias, True),
            _ref(output, True), ctypes.c_void_p(wptr), ctypes.c_size_t(wbytes), _stream_handle(stream)]
    if events is None:
        st = _lib().qmoe_grouped_matmul(*args)
        where = "qmoe_grouped_matmul"
    else:
        ev = (ctypes.c_void_p * QMOE_GMM_EVENTS)()
        for i, e in enumerate(events):
            ev[i] = e
        st = _lib().qmoe_grouped_matmul_debug(*args, ev)
        where = "qmoe_grouped_matmul_debug"
    if st != 0:
        raise QmoeError(st, where)


def grouped_matmul(input, weights, group_indices, bias=None, stream=None, workspace=None, output=None):
    """Allocate output [M, S, N] (and workspace unless given) with torch, then qmoe_grouped_matmul."""
    import torch
    if output is None:
        output = torch.empty((input.shape[0], group_indices.shape[1], weights.shape[2]), dtype=input.dtype,
                             device=input.device)
    need = qmoe_grouped_matmul_workspace_size(input, weights, group_indices, bias, output)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=input.device)
    qmoe_grouped_matmul(input, weights, group_indices, bias, output, workspace, stream)
    return output


qmoe_grouped_matmul_debug = qmoe_grouped_matmul


# ------------------------------------------------------------------ float MoE
MOE_TENSORS = ("input", "router_probs", "fc1_experts_weights", "fc1_experts_bias", "fc2_experts_weights",
               "fc2_experts_bias", "fc3_experts_weights", "fc3_experts_bias")


def qmoe_moe_attrs_default() -> QmoeMoeAttrs:
    a = QmoeMoeAttrs()
    _lib().qmoe_moe_attrs_default(ctypes.byref(a))
    return a


def make_moe_attrs(attrs: Optional[dict] = None) -> QmoeMoeAttrs:
    """qmoe_moe_attrs from a dict of the README's attribute names."""
    a = qmoe_moe_attrs_default()
    for key, val in (attrs or {}).items():
        if key == "activation_type" and isinstance(val, str):
            val = QMOE_ACT.get(val, 99)
        elif key == "swiglu_limit":
            a.has_swiglu_limit = 0 if val is None else 1
            val = 0.0 if val is None else val
        setattr(a, key, val)
    return a


def _moe_refs(ts, data):
    """Eight tensor arguments in C order from a dict (missing = NULL)."""
    return [_ref(ts.get(n), data) for n in MOE_TENSORS]


def _moe_a(attrs):
    return attrs if isinstance(attrs, QmoeMoeAttrs) else make_moe_attrs(attrs)


def qmoe_moe_validate(tensors: dict, attrs=None, output=None) -> int:
    """Status code of the float MoE contract check.  Arrays may live anywhere."""
    a = _moe_a(attrs)
    return int(_lib().qmoe_moe_validate(*_moe_refs(tensors, False), _ref(output, False), ctypes.byref(a)))


def qmoe_moe_workspace_size(tensors: dict, attrs=None) -> int:
    a = _moe_a(attrs)
    n = ctypes.c_size_t(0)
    st = _lib().qmoe_moe_workspace_size(*_moe_refs(tensors, False), ctypes.byref(a), ctypes.byref(n))
    if st != 0:
        raise QmoeError(st, "qmoe_moe_workspace_size")
    return int(n.value)


def qmoe_moe_forward(tensors: dict, attrs, output, workspace, stream=None, debug: Optional[dict] = None) -> None:
    """Enqueue the float MoE on ``stream``.  ``tensors`` maps the names of
    MOE_TENSORS to contiguous device tensors (optional ones may be absent);
    ``debug`` as for qmoe_forward."""
    a = _moe_a(attrs)
    wptr = workspace.data_ptr() if workspace is not None and workspace.numel() > 0 else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = [*_moe_refs(tensors, True), ctypes.byref(a), _ref(output, True), ctypes.c_void_p(wptr),
            ctypes.c_size_t(wbytes), _stream_handle(stream)]
    if debug is None:
        st = _lib().qmoe_moe_forward(*args)
        where = "qmoe_moe_forward"
    else:
        dbg = QmoeDebug()
        for f in ("topk_idx", "topk_w", "counts", "offsets", "perm"):
            t = debug.get(f)
            setattr(dbg, f, t.data_ptr() if t is not None and t.numel() > 0 else None)
        for i, ev in enumerate(debug.get("events") or ()):
            dbg.events[i] = ev
        st = _lib().qmoe_moe_forward_debug(*args, ctypes.byref(dbg))
        where = "qmoe_moe_forward_debug"
    if st != 0:
        raise QmoeError(st, where)


qmoe_moe_forward_debug = qmoe_moe_forward


def moe_forward(tensors: dict, attrs=None, stream=None, workspace=None, output=None, debug=None):
    """Allocate output (and workspace unless given) with torch, then qmoe_moe_forward."""
    import torch
    x = tensors["input"]
    if output is None:
        output = torch.empty_like(x)
    need = qmoe_moe_workspace_size(tensors, attrs)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    qmoe_moe_forward(tensors, attrs, output, workspace, stream, debug)
    return output
