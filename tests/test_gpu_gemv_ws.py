"""GPU parity of qmv_gemv_ws (the split-k lookup-table GEMV of the additive formats at batch 1)
against the CPU oracle, through the C ABI.

Bar as for qmv_gemv: every output within 2e-3 * sum_k |w||x| of the oracle's double result.
Also: an exactly cancelling code pair gives exactly 0, one workspace serves calls of other
shapes in turn, the result is bit-identical across calls, x = e_j returns the weight column to
one rounding, and shapes without a lookup kernel run qmv_gemv unchanged.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_parity, qweights, x_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qmv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_weight_quantized_dequant_amd as q
    q.lib()
    return q


def lut_label(fmt):
    return ("aq2x8" if fmt == synth.FMT_AQ2X8 else "aq3x8") + ".lut-dot.split-k"


def run_ws(qmv, fmt, n, k, xt, seed, ws=None, rows=None):
    import torch
    w = synth.gen_weights(fmt, n, k, seed=seed)
    x = synth.gen_x(1, k, xt, seed=seed)
    print(f"case fmt={fmt} n={n} k={k} xt={xt} seed={seed}", flush=True)
    W = qweights(fmt, n, k, w)
    if ws is None:
        ws = qmv.gemv_workspace(W, 1)
    y = qmv.gemv_ws(W, x_to_device(x, xt), ws)
    torch.cuda.synchronize()
    assert qmv.last_path() == lut_label(fmt)
    y = y.cpu().numpy()
    om = oracle.Mat(fmt, n, k, w)
    yr, b = oracle.gemv(om, x, xt, rows=rows, nthreads=oracle.max_threads())
    return assert_parity(y if rows is None else y[:, rows], yr, b, f"fmt={fmt} {n}x{k} ws")


FMTS = [synth.FMT_AQ2X8, synth.FMT_AQ3X8]
SMALL = [(1, 256), (37, 512), (511, 1024), (513, 256), (1500, 4096 + 256), (3000, 2048), (64, 14336)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", SMALL)
def test_lut_small_full_parity(qmv, fmt, n, k):
    # row counts that leave the last 512-row chunk ragged; one slice (k = 256) through many
    run_ws(qmv, fmt, n, k, synth.DT_BF16, seed=n + k)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xt", [synth.DT_F32, synth.DT_BF16])
def test_lut_dtypes(qmv, fmt, xt):
    run_ws(qmv, fmt, 777, 2048 + 512, xt, seed=11)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 14336)])
def test_lut_config_shapes_all_rows(qmv, fmt, n, k):
    run_ws(qmv, fmt, n, k, synth.DT_BF16, seed=0)


@pytest.mark.parametrize("fmt", FMTS)
def test_lut_aq3_odd_slices(qmv, fmt):
    # k a multiple of 128 but not of 256: AQ3X8 keeps the lookup kernel, AQ2X8 runs qmv_gemv
    import torch
    n, k = 300, 128 * 11
    W = qweights(fmt, n, k, synth.gen_weights(fmt, n, k, seed=2))
    need = qmv.gemv_workspace_bytes(W, 1)
    assert (need > 0) == (fmt == synth.FMT_AQ3X8)
    if fmt == synth.FMT_AQ3X8:
        run_ws(qmv, fmt, n, k, synth.DT_F32, seed=2)
    else:
        x = x_to_device(synth.gen_x(1, k, synth.DT_F32, seed=2), synth.DT_F32)
        y = qmv.gemv_ws(W, x, None)
        torch.cuda.synchronize()
        assert qmv.last_path().startswith("aq2x8.stream")


def test_lut_repeated_calls_share_a_workspace(qmv):
    # one workspace, sized for the largest call, serves calls of other shapes in turn; it
    # starts out holding garbage, which no call may read
    fmt = synth.FMT_AQ2X8
    big = qweights(fmt, 4096, 4096, synth.gen_weights(fmt, 4096, 4096, seed=3))
    ws = qmv.gemv_workspace(big, 1)
    ws.fill_(0xFF)
    for n, k, seed in [(4096, 4096, 3), (1000, 2048, 4), (4096, 4096, 3), (3, 256, 5), (2049, 1024, 6)]:
        run_ws(qmv, fmt, n, k, synth.DT_BF16, seed=seed, ws=ws)


def test_lut_bit_identical_across_calls(qmv):
    # the partials are added in slice order by whichever workgroup finishes last
    import torch
    fmt, n, k = synth.FMT_AQ2X8, 14336, 4096
    W = qweights(fmt, n, k, synth.gen_weights(fmt, n, k, seed=8))
    x = x_to_device(synth.gen_x(1, k, synth.DT_BF16, seed=8), synth.DT_BF16)
    ws = qmv.gemv_workspace(W, 1)
    ys = [qmv.gemv_ws(W, x, ws).clone() for _ in range(5)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


@pytest.mark.parametrize("fmt", FMTS)
def test_lut_cancelling_codebooks_give_zero(qmv, fmt):
    # C2 = -C1 and c2 == c1: every table pair cancels exactly, so the rows come out as 0
    import torch
    n, k = 700, 4096
    w = synth.gen_weights(fmt, n, k, seed=5)
    w["cbk"][1] = -w["cbk"][0]
    w["codes"][:, :, 1] = w["codes"][:, :, 0]
    if fmt == synth.FMT_AQ3X8:
        w["cbk"][2] = 0
    W = qweights(fmt, n, k, w)
    x = x_to_device(synth.gen_x(1, k, synth.DT_BF16, seed=5), synth.DT_BF16)
    y = qmv.gemv_ws(W, x, qmv.gemv_workspace(W, 1))
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0.0)


def test_lut_unit_vector_returns_column(qmv):
    # x = e_j: the table entries of group j/8 are C_b[c][j % 8] exactly and all others 0, so
    # y[n] = s[n] * (C_1[c_1][j % 8] + C_2[c_2][j % 8]), the oracle's value to one rounding
    import torch
    fmt, n, k = synth.FMT_AQ2X8, 1030, 2048
    w = synth.gen_weights(fmt, n, k, seed=9)
    W = qweights(fmt, n, k, w)
    ws = qmv.gemv_workspace(W, 1)
    om = oracle.Mat(fmt, n, k, w)
    for j in [0, 7, 1029, k - 1]:
        x = np.zeros((1, k), dtype=np.float32)
        x[0, j] = 1.0
        y = qmv.gemv_ws(W, torch.from_numpy(x).cuda(), ws)
        torch.cuda.synchronize()
        yr, b = oracle.gemv(om, x, synth.DT_F32)
        assert_parity(y.cpu().numpy(), yr, b, f"e_{j}", rel=1e-6)


def test_gemv_ws_without_a_lookup_kernel_is_gemv(qmv):
    # formats and batches that need no workspace: the call is qmv_gemv, bit for bit
    import torch
    for fmt, n, k, m in [(synth.FMT_Q4_0, 300, 4096, 1), (synth.FMT_AQ2X8, 300, 4096, 4), (synth.FMT_CB4, 64, 1024, 2)]:
        w = synth.gen_weights(fmt, n, k, seed=1)
        W = qweights(fmt, n, k, w)
        assert qmv.gemv_workspace_bytes(W, m) == 0
        x = x_to_device(synth.gen_x(m, k, synth.DT_BF16, seed=1), synth.DT_BF16)
        y0 = qmv.gemv(W, x)
        p0 = qmv.last_path()
        y1 = qmv.gemv_ws(W, x, None)
        torch.cuda.synchronize()
        assert qmv.last_path() == p0
        assert torch.equal(y0, y1)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("scale", [1e-30, 1e-6, 1.0, 3e4, 1e7, 1e30])
def test_lut_activation_magnitudes(qmv, fmt, scale):
    # the tables are built from x scaled by a power of two per slice and split into two fp16
    # halves: activations far outside fp16's range, a slice of zeros and a slice whose values
    # span many binades must all stay within the bound
    import torch
    n, k = 600, 2048
    w = synth.gen_weights(fmt, n, k, seed=21)
    x = synth.gen_x(1, k, synth.DT_F32, seed=21) * np.float32(scale)
    x[0, 256:512] = 0.0                                    # an all-zero slice
    x[0, 512:768] *= np.logspace(-6, 6, 256).astype(np.float32)  # one slice over 12 decades
    x = x.astype(np.float32)
    W = qweights(fmt, n, k, w)
    y = qmv.gemv_ws(W, torch.from_numpy(x).cuda(), qmv.gemv_workspace(W, 1))
    torch.cuda.synchronize()
    yr, b = oracle.gemv(oracle.Mat(fmt, n, k, w), x, synth.DT_F32, nthreads=oracle.max_threads())
    assert_parity(y.cpu().numpy(), yr, b, f"fmt={fmt} x scale {scale:g}")
