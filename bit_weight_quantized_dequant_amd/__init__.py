"""qmv -- fused dequantize-and-multiply of block-quantized weights on MI355X (gfx950).

A thin ctypes binding over libqmv.so, whose C ABI is declared in include/qmv.h.
This module only marshals arguments: every step of the computation runs in the
library's HIP kernels.  PyTorch is used for device memory and the current stream.
If libqmv.so is missing the binding raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import weakref

__all__ = [
    "Q4_0", "Q6_K", "CB4", "AQ2X8", "CB8", "AQ3X8", "F32", "BF16", "QmvError", "QWeights", "lib", "plane_bytes",
    "weight_bytes", "validate", "gemv", "gemv_workspace_bytes", "gemv_workspace", "gemv_ws", "dequant", "quant_act", "workspace_bytes", "gemm",
    "gemm_q8", "gemm_ws", "gemm_noalloc", "partials", "plane_bytes_of", "register_plane", "unregister_plane", "moe_ffn", "last_path",
    "strerror", "PLANES",
]

Q4_0, Q6_K, CB4, AQ2X8, CB8, AQ3X8 = 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1
MAX_BATCH = 8

# Plane names per format, in the order of the descriptor fields they fill.
PLANES = {
    Q4_0: {"qs": "codes", "d": "scales"},
    Q6_K: {"ql": "codes", "qh": "codes_hi", "sc": "scales", "d": "super"},
    CB4: {"idx": "codes", "cb": "codebook"},
    AQ2X8: {"codes": "codes", "s": "scales", "cbk": "codebook"},
    CB8: {"idx": "codes", "cb": "codebook"},
    AQ3X8: {"codes": "codes", "s": "scales", "cbk": "codebook"},
}
_PLANE_ID = {"codes": 0, "codes_hi": 1, "scales": 2, "super": 3, "codebook": 4}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmv.so")


class QmvError(RuntimeError):
    def __init__(self, code: int, call: str):
        self.code = code
        super().__init__(f"{call}: {strerror(code)} ({code})")


class _W(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("n", C.c_int64), ("k", C.c_int64), ("codes", C.c_void_p),
                ("codes_hi", C.c_void_p), ("scales", C.c_void_p), ("super", C.c_void_p),
                ("codebook", C.c_void_p)]


_lib = None


def lib():
    """Load libqmv.so (built in-tree by build.py); raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqmv.so not built ({LIB_PATH}); run "
                              "`python bit_weight_quantized_dequant_amd/build.py`")
        # torch carries its own HIP and HSA runtimes: loaded first, they are the ones the
        # library binds to (its libamdhip64 dependency resolves to the library already in
        # the process).  Loaded after the library, a second HSA runtime would start and the
        # two would not share devices, memory or streams.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        P, I32, I64 = C.c_void_p, C.c_int32, C.c_int64
        L.qmv_plane_bytes.restype = I64
        L.qmv_plane_bytes.argtypes = [I32, I64, I64, I32]
        L.qmv_weight_bytes.restype = I64
        L.qmv_weight_bytes.argtypes = [I32, I64, I64]
        L.qmv_validate.restype = C.c_int
        L.qmv_validate.argtypes = [P, I32, I32]
        L.qmv_gemv.restype = C.c_int
        L.qmv_gemv.argtypes = [P, I32, P, I32, P, P]
        L.qmv_gemv_workspace_bytes.restype = I64
        L.qmv_gemv_workspace_bytes.argtypes = [P, I32]
        L.qmv_gemv_ws.restype = C.c_int
        L.qmv_gemv_ws.argtypes = [P, I32, P, I32, P, P, I64, P]
        L.qmv_gemv_q8.restype = C.c_int
        L.qmv_read_ceiling.restype = C.c_int
        L.qmv_read_ceiling.argtypes = [P, I64, P, P]
        L.qmv_gemv_q8.argtypes = [P, I32, P, P, P, P]
        L.qmv_dequant.restype = C.c_int
        L.qmv_dequant.argtypes = [P, P, P]
        L.qmm_quant_act.restype = C.c_int
        L.qmm_quant_act.argtypes = [P, I32, I64, P, P, P]
        L.qmm_workspace_bytes.restype = I64
        L.qmm_workspace_bytes.argtypes = [P, I32]
        L.qmm_gemm.restype = C.c_int
        L.qmm_gemm.argtypes = [P, I32, P, P, P, I64, P]
        L.qmm_gemm_q8.restype = C.c_int
        L.qmm_gemm_q8.argtypes = [P, I32, P, P, P, P]
        L.qmm_partials.restype = C.c_int
        L.qmm_partials.argtypes = [P, I32, P, P, P]
        L.qmm_gemm_ws.restype = C.c_int
        L.qmm_gemm_ws.argtypes = [P, I32, P, I64, P, P]
        L.qmm_gemm_noalloc.restype = C.c_int
        L.qmm_gemm_noalloc.argtypes = [P, I32, P, P, P]
        L.qmm_plane_bytes.restype = I64
        L.qmm_plane_bytes.argtypes = [P]
        L.qmm_register_plane.restype = C.c_int
        L.qmm_register_plane.argtypes = [P, P, I64, P]
        L.qmm_unregister_plane.restype = C.c_int
        L.qmm_unregister_plane.argtypes = [P]
        L.qmv_moe_ffn.restype = C.c_int
        L.qmv_moe_ffn.argtypes = [P, P, P, I32, P, I32, P, I32, P, P, P]
        L.qmv_last_path.restype = C.c_char_p
        L.qmv_last_path.argtypes = []
        L.qmv_strerror.restype = C.c_char_p
        L.qmv_strerror.argtypes = [C.c_int]
        L.qmv_version.restype = C.c_char_p
        L.qmv_version.argtypes = []
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().qmv_strerror(code).decode()


def last_path() -> str:
    return lib().qmv_last_path().decode()


def plane_bytes(fmt: int, n: int, k: int, plane: str) -> int:
    return lib().qmv_plane_bytes(fmt, n, k, _PLANE_ID[plane])


def weight_bytes(fmt: int, n: int, k: int) -> int:
    return lib().qmv_weight_bytes(fmt, n, k)


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


class QWeights:
    """A quantized matrix on the device: format, shape and its plane tensors.

    `planes` maps the format's plane names (see PLANES) to device tensors (or raw
    integer device addresses).  The object keeps references to them.
    """

    def __init__(self, fmt: int, n: int, k: int, planes: dict):
        self.fmt, self.n, self.k = fmt, n, k
        self.planes = dict(planes)
        fields = {f: 0 for f in ("codes", "codes_hi", "scales", "super", "codebook")}
        for name, field in PLANES[fmt].items():
            t = self.planes.get(name)
            if t is not None and not isinstance(t, int):
                if not t.is_cuda or not t.is_contiguous():
                    raise ValueError(f"plane {name}: must be a contiguous device tensor")
                need = plane_bytes(fmt, n, k, field)
                if need > 0 and t.numel() * t.element_size() < need:
                    raise ValueError(f"plane {name}: {t.numel() * t.element_size()} bytes, "
                                     f"the format needs {need}")
            fields[field] = _ptr(t)
        self._s = _W(fmt, n, k, *(fields[f] for f in ("codes", "codes_hi", "scales", "super", "codebook")))

    @property
    def ref(self):
        return C.byref(self._s)

    def nbytes(self) -> int:
        return weight_bytes(self.fmt, self.n, self.k)


def _check(rc: int, call: str):
    if rc != 0:
        raise QmvError(rc, call)


def _need(t, dtypes, shape, name: str):
    """Check a tensor argument before its address is handed to the library: the C ABI sees
    only a pointer, so a wrong dtype, shape or layout would be read or written as if it were
    right.  Raw integer addresses are passed through unchecked."""
    if isinstance(t, int):
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def validate(w: QWeights, m: int = 1, xt: int = F32) -> int:
    return lib().qmv_validate(w.ref, m, xt)


def _xt_of(x) -> int:
    import torch
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {x.dtype}")


def gemv(w: QWeights, x, y=None, stream=None):
    """y[m][n] = W x[m] for x of shape [m][k] (or [k]); returns y (fp32)."""
    import torch
    squeeze = x.dim() == 1
    x2 = x.reshape(1, -1) if squeeze else x
    m = x2.shape[0]
    _need(x2, (torch.float32, torch.bfloat16), (m, w.k), "x")
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=x.device)
    _need(y, (torch.float32,), (m, w.n), "y")
    _check(lib().qmv_gemv(w.ref, m, _ptr(x2), _xt_of(x2), _ptr(y), _stream(stream)), "qmv_gemv")
    return y[0] if squeeze else y


def gemv_workspace_bytes(w: QWeights, m: int = 1) -> int:
    """qmv_gemv_workspace_bytes: bytes of the workspace gemv_ws needs for (w, m); 0 if none."""
    need = lib().qmv_gemv_workspace_bytes(w.ref, m)
    if need < 0:
        raise QmvError(need, "qmv_gemv_workspace_bytes")
    return need


def gemv_workspace(w: QWeights, m: int = 1, device="cuda"):
    """A workspace for gemv_ws (uint8 device tensor), or None if none is needed.  One
    workspace serves any number of ordered calls of the same or smaller size."""
    import torch
    need = gemv_workspace_bytes(w, m)
    return torch.empty(need, dtype=torch.uint8, device=device) if need else None


def gemv_ws(w: QWeights, x, ws, y=None, stream=None):
    """qmv_gemv_ws: y[m][n] = W x[m] with the split-k kernels that need the workspace ws (from
    gemv_workspace; None when gemv_workspace_bytes is 0)."""
    import torch
    squeeze = x.dim() == 1
    x2 = x.reshape(1, -1) if squeeze else x
    m = x2.shape[0]
    _need(x2, (torch.float32, torch.bfloat16), (m, w.k), "x")
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=x.device)
    _need(y, (torch.float32,), (m, w.n), "y")
    if ws is not None:
        _need(ws, (torch.uint8,), None, "ws")
    wp, wn = (_ptr(ws), ws.numel()) if ws is not None else (None, 0)
    _check(lib().qmv_gemv_ws(w.ref, m, _ptr(x2), _xt_of(x2), _ptr(y), wp, wn, _stream(stream)), "qmv_gemv_ws")
    return y[0] if squeeze else y


def gemv_q8(w: QWeights, xq, xs, y=None, stream=None):
    """q4_0 or q6_K GEMV over int8 activations (xq int8 [m][k], xs fp32 [m][k/32], as
    quant_act writes them); y fp32 [m][n] is allocated unless given."""
    import torch
    m = xq.shape[0]
    _need(xq, (torch.int8,), (m, w.k), "xq")
    _need(xs, (torch.float32,), (m, w.k // 32), "xs")
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=xq.device)
    _need(y, (torch.float32,), (m, w.n), "y")
    _check(lib().qmv_gemv_q8(w.ref, m, _ptr(xq), _ptr(xs), _ptr(y), _stream(stream)), "qmv_gemv_q8")
    return y


def read_ceiling(t, sink, stream=None):
    """Measurement only: read every byte of device tensor t (contiguous, a multiple of 16
    bytes) and nothing else; sink is a device int32/uint32 tensor of at least one element."""
    import torch
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("t: must be a contiguous device tensor")
    _need(sink, (torch.int32,), None, "sink")
    _check(lib().qmv_read_ceiling(_ptr(t), t.numel() * t.element_size(), _ptr(sink), _stream(stream)),
           "qmv_read_ceiling")


def dequant(w: QWeights, out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((w.n, w.k), dtype=torch.float32, device="cuda")
    _need(out, (torch.float32,), (w.n, w.k), "out")
    _check(lib().qmv_dequant(w.ref, _ptr(out), _stream(stream)), "qmv_dequant")
    return out


def quant_act(x, xq=None, xs=None, stream=None):
    import torch
    m, k = x.shape
    _need(x, (torch.float32,), (m, k), "x")
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    _need(xq, (torch.int8,), (m, k), "xq")
    _need(xs, (torch.float32,), (m, k // 32), "xs")
    _check(lib().qmm_quant_act(_ptr(x), m, k, _ptr(xq), _ptr(xs), _stream(stream)), "qmm_quant_act")
    return xq, xs


def workspace_bytes(w: QWeights, m: int) -> int:
    return lib().qmm_workspace_bytes(w.ref, m)


def gemm(w: QWeights, x, y=None, ws=None, stream=None):
    import torch
    m = x.shape[0]
    _need(x, (torch.float32,), (m, w.k), "x")
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=x.device)
    _need(y, (torch.float32,), (m, w.n), "y")
    need = workspace_bytes(w, m)
    if need < 0:
        raise QmvError(need, "qmm_workspace_bytes")
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    _need(ws, (torch.uint8,), None, "ws")
    _check(lib().qmm_gemm(w.ref, m, _ptr(x), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)), "qmm_gemm")
    return y


def gemm_ws(w: QWeights, ws, y=None, m=None, stream=None):
    """qmm_gemm_ws: the contraction alone, on the activations a previous gemm() with the same
    m and k quantized into ws (uint8 device tensor); y fp32 [m][n] allocated unless given."""
    import torch
    if m is None:
        m = y.shape[0]
    _need(ws, (torch.uint8,), None, "ws")
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=ws.device)
    _need(y, (torch.float32,), (m, w.n), "y")
    _check(lib().qmm_gemm_ws(w.ref, m, _ptr(ws), ws.numel(), _ptr(y), _stream(stream)), "qmm_gemm_ws")
    return y


def gemm_noalloc(w: QWeights, x, y, stream=None):
    """qmm_gemm_noalloc: the q6_K GEMM with the library's own per-GPU scratch instead of a
    workspace; y (fp32 [m][n]) must be given, nothing is allocated."""
    import torch
    m = x.shape[0]
    _need(x, (torch.float32,), (m, w.k), "x")
    _need(y, (torch.float32,), (m, w.n), "y")
    _check(lib().qmm_gemm_noalloc(w.ref, m, _ptr(x), _ptr(y), _stream(stream)), "qmm_gemm_noalloc")
    return y


def gemm_q8(w: QWeights, xq, xs, y=None, stream=None):
    import torch
    m = xq.shape[0]
    _need(xq, (torch.int8,), (m, w.k), "xq")
    _need(xs, (torch.float32,), (m, w.k // 32), "xs")
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=xq.device)
    _need(y, (torch.float32,), (m, w.n), "y")
    _check(lib().qmm_gemm_q8(w.ref, m, _ptr(xq), _ptr(xs), _ptr(y), _stream(stream)), "qmm_gemm_q8")
    return y


def partials(w: QWeights, xq, out=None, stream=None):
    import torch
    m = xq.shape[0]
    _need(xq, (torch.int8,), (m, w.k), "xq")
    if out is None:
        out = torch.empty((m, w.n, w.k // 32), dtype=torch.int32, device=xq.device)
    _need(out, (torch.int32,), (m, w.n, w.k // 32), "out")
    _check(lib().qmm_partials(w.ref, m, _ptr(xq), _ptr(out), _stream(stream)), "qmm_partials")
    return out


def plane_bytes_of(w: QWeights) -> int:
    return lib().qmm_plane_bytes(w.ref)


def _forget_plane(desc, plane):
    # finalizer of a registered QWeights: drop the library's record before the plane's
    # memory (and the codes' memory, which keys the record) can be reused by another matrix
    lib().qmm_unregister_plane(C.byref(desc))


def register_plane(w: QWeights, plane=None, stream=None):
    """Fill a pre-expanded plane for the q6_K GEMM (allocated here unless given) and record
    it for w.  The plane is kept alive with w; when w is garbage-collected (or
    unregister_plane is called) the library's record is dropped, so a later matrix whose
    tensors reuse the same addresses never picks up a stale plane.  Returns the plane."""
    import torch
    need = plane_bytes_of(w)
    if need < 0:
        raise QmvError(need, "qmm_plane_bytes")
    if plane is None:
        plane = torch.empty(need, dtype=torch.uint8, device="cuda")
    _need(plane, (plane.dtype,), None, "plane")
    _check(lib().qmm_register_plane(w.ref, _ptr(plane), plane.numel() * plane.element_size(), _stream(stream)),
           "qmm_register_plane")
    old = getattr(w, "_plane_fin", None)
    if old is not None:
        old.detach()
    desc = _W(w._s.fmt, w._s.n, w._s.k, w._s.codes, w._s.codes_hi, w._s.scales, w._s.super, w._s.codebook)
    w._plane_fin = weakref.finalize(w, _forget_plane, desc, plane)
    return plane


def unregister_plane(w: QWeights):
    _check(lib().qmm_unregister_plane(w.ref), "qmm_unregister_plane")
    fin = getattr(w, "_plane_fin", None)
    if fin is not None:
        fin.detach()
        w._plane_fin = None


def moe_ffn(gate: QWeights, up: QWeights, down: QWeights, n_experts: int, ids, x, h=None, y=None,
            stream=None):
    """Routed-expert FFN for one token: returns (h [n_ids][d_ff], y [n_ids][d_model])."""
    import torch
    n_ids = ids.numel()
    _need(ids, (torch.int32,), (n_ids,), "ids")
    _need(x, (torch.float32, torch.bfloat16), (gate.k,), "x")
    if h is None:
        h = torch.empty((n_ids, gate.n), dtype=torch.float32, device=x.device)
    if y is None:
        y = torch.empty((n_ids, down.n), dtype=torch.float32, device=x.device)
    _need(h, (torch.float32,), (n_ids, gate.n), "h")
    _need(y, (torch.float32,), (n_ids, down.n), "y")
    _check(lib().qmv_moe_ffn(gate.ref, up.ref, down.ref, n_experts, _ptr(ids), n_ids, _ptr(x),
                             _xt_of(x), _ptr(h), _ptr(y), _stream(stream)), "qmv_moe_ffn")
    return h, y
