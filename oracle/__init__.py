"""CPU oracle for the quantized GEMV / GEMM path (ctypes wrapper over qmv_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of
the benchmark are the only callers.  The GPU library never imports, links or runs
anything here, and nothing here imports the GPU library.

Every function decodes stored codes to exact integers, forms weights exactly and
accumulates in double (see qmv_oracle.c for the readings of each layout).  The
mixture-of-experts composition below follows the workload description: for each
routed expert, h = SiLU(gate x) * (up x), then y = down h; SiLU(z) = z/(1+e^-z).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

Q4_0, Q6_K, CB4, AQ2X8, CB8, AQ3X8 = 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1

_PLANES = {Q4_0: ("qs", "d"), Q6_K: ("ql", "qh", "sc", "d"), CB4: ("idx", "cb"),
           AQ2X8: ("codes", "cbk", "s"), CB8: ("idx", "cb"), AQ3X8: ("codes", "cbk", "s")}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction, no fast math, OpenMP over rows)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class _Mat(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("n", C.c_int64), ("k", C.c_int64),
                ("p0", C.c_void_p), ("p1", C.c_void_p), ("p2", C.c_void_p), ("p3", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = C.CDLL(LIB)
        P = C.c_void_p
        I64, I32, D = C.c_int64, C.c_int32, C.c_double
        L.qo_f16.restype = D
        L.qo_f16.argtypes = [C.c_uint16]
        L.qo_bf16.restype = D
        L.qo_bf16.argtypes = [C.c_uint16]
        L.qo_weight.restype = D
        L.qo_weight.argtypes = [P, I64, I64]
        L.qo_dequant.argtypes = [P, P]
        L.qo_codes.argtypes = [P, P]
        L.qo_gemv_rows.argtypes = [P, I32, P, I32, P, I64, P, P, I32]
        L.qo_silu.restype = D
        L.qo_silu.argtypes = [D]
        L.qo_quant_act.argtypes = [P, I64, I64, P, P]
        L.qo_q6k_partials.argtypes = [P, P, P, P, I64, P, P]
        L.qo_q6k_gemm_pairs.argtypes = [P, P, P, P, P, I64, P, P, I32]
        L.qo_q4_0_gemv_q8_pairs.argtypes = [P, P, P, P, P, I64, P, P, I32]
        L.qo_pack_q4_0.argtypes = [P, I64, I64, P]
        L.qo_pack_q6k.argtypes = [P, I64, I64, P, P]
        L.qo_pack_cb4.argtypes = [P, I64, I64, P]
        L.qo_q4_0_to_blocks.argtypes = [P, P, I64, P]
        L.qo_q4_0_from_blocks.argtypes = [P, I64, P, P]
        L.qo_q6k_to_blocks.argtypes = [P, P, P, P, I64, P]
        L.qo_q6k_from_blocks.argtypes = [P, I64, P, P, P, P]
        L.qo_max_threads.restype = I32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


class Mat:
    """A host weight matrix for the oracle: format, shape and its planes."""

    def __init__(self, fmt: int, n: int, k: int, planes: dict):
        self.fmt, self.n, self.k = fmt, n, k
        self.planes = {name: np.ascontiguousarray(planes[name]) for name in _PLANES[fmt]}
        ptrs = [_p(self.planes[name]) for name in _PLANES[fmt]] + [None] * (4 - len(_PLANES[fmt]))
        self._s = _Mat(fmt, n, k, *ptrs)

    @property
    def ref(self):
        return C.byref(self._s)


def f16(bits: int) -> float:
    return lib().qo_f16(bits)


def bf16(bits: int) -> float:
    return lib().qo_bf16(bits)


def weight(m: Mat, row: int, col: int) -> float:
    return lib().qo_weight(m.ref, row, col)


def dequant(m: Mat) -> np.ndarray:
    w = np.empty((m.n, m.k), dtype=np.float64)
    lib().qo_dequant(m.ref, _p(w))
    return w


def codes(m: Mat) -> np.ndarray:
    out = np.empty((m.n, m.k), dtype=np.int32)
    lib().qo_codes(m.ref, _p(out))
    return out


def gemv(m: Mat, x: np.ndarray, xt: int = F32, rows=None, nthreads: int = 1):
    """(y, bound), each float64 [batch][len(rows) or n]."""
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x[None, :]
    assert x.shape[1] == m.k and x.dtype == (np.float32 if xt == F32 else np.uint16)
    batch = x.shape[0]
    if rows is None:
        nr, rp = m.n, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nr, rp = len(rows), _p(rows)
    y = np.empty((batch, nr), dtype=np.float64)
    b = np.empty((batch, nr), dtype=np.float64)
    lib().qo_gemv_rows(m.ref, batch, _p(x), xt, rp, nr, _p(y), _p(b), nthreads)
    return y, b


def silu(z: float) -> float:
    return lib().qo_silu(float(z))


def quant_act(x: np.ndarray):
    """Per-32 int8 activation quantizer: (xq int8 [m][k], xs float32 [m][k/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    mr, k = x.shape
    assert k % 32 == 0
    xq = np.empty((mr, k), dtype=np.int8)
    xs = np.empty((mr, k // 32), dtype=np.float32)
    lib().qo_quant_act(_p(x), mr, k, _p(xq), _p(xs))
    return xq, xs


def q6k_partials(m: Mat, xq: np.ndarray, mm, nn):
    """Exact P16 [pair][k/16] and I32 [pair][k/32] (int64) for (mm[i], nn[i]) pairs."""
    mm = np.ascontiguousarray(mm, dtype=np.int64)
    nn = np.ascontiguousarray(nn, dtype=np.int64)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    p16 = np.empty((len(mm), m.k // 16), dtype=np.int64)
    i32 = np.empty((len(mm), m.k // 32), dtype=np.int64)
    lib().qo_q6k_partials(m.ref, _p(xq), _p(mm), _p(nn), len(mm), _p(p16), _p(i32))
    return p16, i32


def q6k_gemm_pairs(m: Mat, xq: np.ndarray, xs: np.ndarray, mm, nn, nthreads: int = 1):
    """(y, bound) float64 [pair] of the q6_K int8 GEMM for (mm[i], nn[i]) pairs."""
    mm = np.ascontiguousarray(mm, dtype=np.int64)
    nn = np.ascontiguousarray(nn, dtype=np.int64)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    y = np.empty(len(mm), dtype=np.float64)
    b = np.empty(len(mm), dtype=np.float64)
    lib().qo_q6k_gemm_pairs(m.ref, _p(xq), _p(xs), _p(mm), _p(nn), len(mm), _p(y), _p(b), nthreads)
    return y, b


def q6k_gemm(m: Mat, x: np.ndarray, nthreads: int = 1):
    """Full q6_K GEMM y [M][N] (quantizer included): (y, bound, xq, xs)."""
    xq, xs = quant_act(x)
    M = xq.shape[0]
    mm, nn = np.meshgrid(np.arange(M), np.arange(m.n), indexing="ij")
    y, b = q6k_gemm_pairs(m, xq, xs, mm.ravel(), nn.ravel(), nthreads)
    return y.reshape(M, m.n), b.reshape(M, m.n), xq, xs


def q4_0_gemv_q8_pairs(m: Mat, xq: np.ndarray, xs: np.ndarray, mm, nn, nthreads: int = 1):
    """(y, bound) float64 [pair] of the q4_0 GEMV over int8 activations (xq, xs from
    quant_act) for (mm[i], nn[i]) pairs: per block d * xs * exact sum of (q - 8) * xq."""
    mm = np.ascontiguousarray(mm, dtype=np.int64)
    nn = np.ascontiguousarray(nn, dtype=np.int64)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    y = np.empty(len(mm), dtype=np.float64)
    b = np.empty(len(mm), dtype=np.float64)
    lib().qo_q4_0_gemv_q8_pairs(m.ref, _p(xq), _p(xs), _p(mm), _p(nn), len(mm), _p(y), _p(b), nthreads)
    return y, b


def q4_0_gemv_q8(m: Mat, xq: np.ndarray, xs: np.ndarray, rows=None, nthreads: int = 1):
    """(y, bound) float64 [M][rows] of the q4_0 GEMV over int8 activations, for all batch
    rows and the listed weight rows (all rows when None)."""
    M = xq.shape[0]
    rows = np.arange(m.n) if rows is None else np.asarray(rows, dtype=np.int64)
    mm, nn = np.meshgrid(np.arange(M), rows, indexing="ij")
    y, b = q4_0_gemv_q8_pairs(m, xq, xs, mm.ravel(), nn.ravel(), nthreads)
    return y.reshape(M, len(rows)), b.reshape(M, len(rows))


def moe_gateup(gate: Mat, up: Mat, x: np.ndarray, xt: int, rows=None, nthreads: int = 1):
    """One expert's first stage: g = gate x, u = up x, h = SiLU(g) * u (double)."""
    g, bg = gemv(gate, x, xt, rows, nthreads)
    u, bu = gemv(up, x, xt, rows, nthreads)
    g, u, bg, bu = g[0], u[0], bg[0], bu[0]
    sg = np.array([silu(v) for v in g])
    return sg * u, g, u, bg, bu


def pack_q4_0(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int32)
    n, k = q.shape
    qs = np.empty((n, k // 32, 16), dtype=np.uint8)
    lib().qo_pack_q4_0(_p(q), n, k, _p(qs))
    return qs


def pack_q6k(q: np.ndarray):
    q = np.ascontiguousarray(q, dtype=np.int32)
    n, k = q.shape
    ql = np.empty((n, k // 256, 128), dtype=np.uint8)
    qh = np.empty((n, k // 256, 64), dtype=np.uint8)
    lib().qo_pack_q6k(_p(q), n, k, _p(ql), _p(qh))
    return ql, qh


def pack_cb4(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int32)
    n, k = q.shape
    idx = np.empty((n, k // 2), dtype=np.uint8)
    lib().qo_pack_cb4(_p(q), n, k, _p(idx))
    return idx


def q4_0_to_blocks(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    nb = d.size
    out = np.empty(nb * 18, dtype=np.uint8)
    lib().qo_q4_0_to_blocks(_p(np.ascontiguousarray(qs)), _p(np.ascontiguousarray(d).view(np.uint16)), nb, _p(out))
    return out


def q4_0_from_blocks(blk: np.ndarray):
    nb = blk.size // 18
    qs = np.empty(nb * 16, dtype=np.uint8)
    d = np.empty(nb, dtype=np.uint16)
    lib().qo_q4_0_from_blocks(_p(np.ascontiguousarray(blk)), nb, _p(qs), _p(d))
    return qs, d.view(np.float16)


def q6k_to_blocks(ql, qh, sc, d) -> np.ndarray:
    ns = d.size
    out = np.empty(ns * 210, dtype=np.uint8)
    lib().qo_q6k_to_blocks(_p(np.ascontiguousarray(ql)), _p(np.ascontiguousarray(qh)),
                           _p(np.ascontiguousarray(sc)), _p(np.ascontiguousarray(d).view(np.uint16)),
                           ns, _p(out))
    return out


def q6k_from_blocks(blk: np.ndarray):
    ns = blk.size // 210
    ql = np.empty(ns * 128, dtype=np.uint8)
    qh = np.empty(ns * 64, dtype=np.uint8)
    sc = np.empty(ns * 16, dtype=np.int8)
    d = np.empty(ns, dtype=np.uint16)
    lib().qo_q6k_from_blocks(_p(np.ascontiguousarray(blk)), ns, _p(ql), _p(qh), _p(sc), _p(d))
    return ql, qh, sc, d.view(np.float16)


def max_threads() -> int:
    return lib().qo_max_threads()
