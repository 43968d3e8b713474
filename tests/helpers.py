"""Shared test helpers: device upload of synthetic planes and the parity criterion."""
import numpy as np

import synth

PLANES = {synth.FMT_Q4_0: ("qs", "d"), synth.FMT_Q6_K: ("ql", "qh", "sc", "d"),
          synth.FMT_CB4: ("idx", "cb"), synth.FMT_AQ2X8: ("codes", "cbk", "s"),
          synth.FMT_CB8: ("idx", "cb"), synth.FMT_AQ3X8: ("codes", "cbk", "s")}

# Per-element bound on |y_gpu - y_ref|, relative to sum_k |w||x| (the stated float tolerance).
REL_TOL = 2e-3


def to_device(planes: dict):
    import torch
    out = {}
    for name, a in planes.items():
        a = np.ascontiguousarray(a)
        if a.dtype == np.float16:
            t = torch.from_numpy(a.view(np.uint16).copy()).view(torch.float16)
        else:
            t = torch.from_numpy(a.copy())
        out[name] = t.cuda()
    return out


def qweights(fmt, n, k, planes):
    import bit_weight_quantized_dequant_amd as qmv
    return qmv.QWeights(fmt, n, k, to_device(planes))


def x_to_device(x: np.ndarray, xt: int):
    import torch
    if xt == synth.DT_F32:
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16).copy()).view(torch.bfloat16).cuda()


def assert_parity(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what: str = "", rel=REL_TOL):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    err = np.abs(y_gpu - y_ref)
    lim = rel * bound
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; worst at {i}: "
                             f"gpu={y_gpu[i]!r} ref={y_ref[i]!r} bound={bound[i]!r}")
    return float(np.max(err / np.where(bound > 0, bound, 1.0)))
