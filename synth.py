"""Seeded synthetic inputs for the quantized GEMV / GEMM workloads.

This module draws the stored bytes of every weight plane and the activations.
It holds none of the method's arithmetic: packed code planes are drawn as
uniform random bytes (a uniform byte is a uniform pair of 4-bit fields, four
uniform 2-bit fields, or one uniform 8-bit code, so every packed field comes out
uniform and independent without any packing step), and scales / codebooks are
drawn as floats and rounded to their storage type.  Both the GPU path and the
CPU oracle take their inputs from here and from nowhere else.

Plane shapes (row-major, rows = output features n, columns = input features k):

  q4_0    qs u8 [N][K/32][16]   d f16 [N][K/32]
  q6_K    ql u8 [N][K/256][128] qh u8 [N][K/256][64] sc i8 [N][K/256][16] d f16 [N][K/256]
  cb4     idx u8 [N][K/2]       cb f16 [N][K/128][16]
  aq2x8   codes u8 [N][K/8][2]  cbk f16 [2][256][8]  s f16 [N]
  cb8     idx u8 [N][K]         cb f16 [N][256]
  aq3x8   codes u8 [N][K/8][3]  cbk f16 [3][256][8]  s f16 [N]

Value distributions follow the workload descriptions: q4_0 d = 0.02*U(0.5,1.5)/8;
q6_K sc ~ U{1..127}, d = 1e-4*U(0.5,1.5); cb4 entries = sorted draws of N(0, 0.02);
aq2x8 and aq3x8 codebooks N(0, 0.01), row scale U(0.5, 1.5); cb8 entries = sorted draws
of N(0, 0.02) (the cb4 distribution, 256 per row); activations N(0, 1).
N(0, s) means standard deviation s.

Every plane has its own stream: SeedSequence([seed, tag, plane, extra...]) fed to
PCG64DXSM, so a plane can be regenerated without drawing the others.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "FMT_Q4_0", "FMT_Q6_K", "FMT_CB4", "FMT_AQ2X8", "FMT_CB8", "FMT_AQ3X8",
    "DT_F32", "DT_BF16",
    "gen_weights", "gen_x", "gen_moe_ids", "rand_bytes", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "plane_names",
]

FMT_Q4_0, FMT_Q6_K, FMT_CB4, FMT_AQ2X8, FMT_CB8, FMT_AQ3X8 = 1, 2, 3, 4, 5, 6
DT_F32, DT_BF16 = 0, 1

_PLANES = {
    FMT_Q4_0: ("qs", "d"),
    FMT_Q6_K: ("ql", "qh", "sc", "d"),
    FMT_CB4: ("idx", "cb"),
    FMT_AQ2X8: ("codes", "cbk", "s"),
    FMT_CB8: ("idx", "cb"),
    FMT_AQ3X8: ("codes", "cbk", "s"),
}


def plane_names(fmt: int):
    return _PLANES[fmt]


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64DXSM(np.random.SeedSequence([int(k) for k in key])))


def rand_bytes(nbytes: int, *key: int) -> np.ndarray:
    """Uniform random bytes, as a flat uint8 array of length nbytes."""
    rng = _rng(*key)
    words = (nbytes + 7) // 8
    raw = rng.bit_generator.random_raw(words)
    return np.ascontiguousarray(raw.view(np.uint8)[:nbytes])


def _f16(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.ascontiguousarray(a, dtype=np.float32))
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = r.astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gen_weights(fmt: int, n: int, k: int, seed: int = 0, expert: int = 0, matrix: int = 0) -> dict:
    """Draw every plane of one n x k weight matrix in format `fmt`.

    `expert` and `matrix` select independent streams so that one expert of a
    mixture (and one of its gate / up / down matrices) can be regenerated alone.
    """
    key = (seed, fmt, expert, matrix)
    if fmt == FMT_Q4_0:
        if k % 32:
            raise ValueError("q4_0 needs k % 32 == 0")
        nb = n * (k // 32)
        qs = rand_bytes(nb * 16, *key, 1).reshape(n, k // 32, 16)
        d = _f16(0.02 * _rng(*key, 2).uniform(0.5, 1.5, nb) / 8).reshape(n, k // 32)
        return {"qs": qs, "d": d}
    if fmt == FMT_Q6_K:
        if k % 256:
            raise ValueError("q6_K needs k % 256 == 0")
        ns = n * (k // 256)
        ql = rand_bytes(ns * 128, *key, 1).reshape(n, k // 256, 128)
        qh = rand_bytes(ns * 64, *key, 2).reshape(n, k // 256, 64)
        sc = _rng(*key, 3).integers(1, 128, ns * 16, dtype=np.int64).astype(np.int8)
        d = _f16(1e-4 * _rng(*key, 4).uniform(0.5, 1.5, ns)).reshape(n, k // 256)
        return {"ql": ql, "qh": qh, "sc": sc.reshape(n, k // 256, 16), "d": d}
    if fmt == FMT_CB4:
        if k % 128:
            raise ValueError("cb4 needs k % 128 == 0")
        ng = n * (k // 128)
        idx = rand_bytes(n * k // 2, *key, 1).reshape(n, k // 2)
        cb = np.sort(_rng(*key, 2).normal(0.0, 0.02, (ng, 16)), axis=1)
        return {"idx": idx, "cb": _f16(cb).reshape(n, k // 128, 16)}
    if fmt in (FMT_AQ2X8, FMT_AQ3X8):
        if k % 8:
            raise ValueError("additive codes need k % 8 == 0")
        nb = 2 if fmt == FMT_AQ2X8 else 3
        codes = rand_bytes(n * (k // 8) * nb, *key, 1).reshape(n, k // 8, nb)
        cbk = _f16(_rng(*key, 2).normal(0.0, 0.01, (nb, 256, 8)))
        s = _f16(_rng(*key, 3).uniform(0.5, 1.5, n))
        return {"codes": codes, "cbk": cbk, "s": s}
    if fmt == FMT_CB8:
        idx = rand_bytes(n * k, *key, 1).reshape(n, k)
        cb = np.sort(_rng(*key, 2).normal(0.0, 0.02, (n, 256)), axis=1)
        return {"idx": idx, "cb": _f16(cb)}
    raise ValueError(f"unknown format {fmt}")


def gen_x(batch: int, k: int, dtype: int = DT_F32, seed: int = 0, stream: int = 0) -> np.ndarray:
    """Activations N(0,1), shape [batch][k]: float32, or bf16 bits as uint16."""
    v = _rng(seed, 100, stream).standard_normal((batch, k)).astype(np.float32)
    if dtype == DT_F32:
        return v
    if dtype == DT_BF16:
        return f32_to_bf16_bits(v)
    raise ValueError("dtype")


def gen_moe_ids(tokens: int, n_experts: int = 256, top: int = 8, seed: int = 0) -> np.ndarray:
    """Per token, `top` distinct expert ids drawn without replacement: int32 [tokens][top]."""
    rng = _rng(seed, 200)
    out = np.empty((tokens, top), dtype=np.int32)
    for t in range(tokens):
        out[t] = rng.choice(n_experts, size=top, replace=False)
    return out
