"""GPU parity of the q6_K prefill GEMM (int8 MFMA) against the CPU oracle.

Bar: the int32 per-block partials I32[m][n][c] are bit-exact; every output is within
2e-3 * sum_k |w| |x_hat| of the oracle's double result (x_hat = xs * xq, the quantized
activations, as the oracle defines the GEMM); full workload sizes are checked on
sampled (m, n) pairs, which the oracle computes one by one.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_parity, qweights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qmv():
    import torch
    assert torch.cuda.is_available()
    import bit_weight_quantized_dequant_amd as q
    q.lib()
    return q


def _setup(qmv, n, k, m, seed):
    import torch
    w = synth.gen_weights(synth.FMT_Q6_K, n, k, seed=seed)
    x = synth.gen_x(m, k, seed=seed)
    print(f"gemm case n={n} k={k} m={m} seed={seed}", flush=True)
    return w, x, qweights(synth.FMT_Q6_K, n, k, w), torch.from_numpy(x).cuda()


@pytest.mark.parametrize("n,k,m", [(32, 256, 32), (64, 512, 128), (70, 768, 45), (130, 1024, 200), (3, 256, 1)])
def test_partials_bit_exact(qmv, n, k, m):
    import torch
    w, x, W, xd = _setup(qmv, n, k, m, seed=n + m)
    xq, xs = qmv.quant_act(xd)
    p = qmv.partials(W, xq)
    torch.cuda.synchronize()
    assert qmv.last_path().endswith(".partials")
    p = p.cpu().numpy()
    rq, _ = oracle.quant_act(x)
    mm, nn = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    _, i32 = oracle.q6k_partials(oracle.Mat(oracle.Q6_K, n, k, w), rq, mm.ravel(), nn.ravel())
    assert np.array_equal(p.reshape(m * n, k // 32).astype(np.int64), i32)


@pytest.mark.parametrize("n,k,m", [(64, 256, 128), (100, 1024, 77), (257, 2048, 130), (128, 4096, 512)])
def test_gemm_full_parity(qmv, n, k, m):
    import torch
    w, x, W, xd = _setup(qmv, n, k, m, seed=n * 3 + m)
    y = qmv.gemm(W, xd)
    torch.cuda.synchronize()
    assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split"
    yr, b, _, _ = oracle.q6k_gemm(oracle.Mat(oracle.Q6_K, n, k, w), x, nthreads=8)
    assert_parity(y.cpu().numpy(), yr, b, f"gemm {n}x{k} m={m}")


@pytest.mark.parametrize("n,k", [(11008, 4096), (4096, 11008)])
def test_gemm_prefill_shapes_sampled(qmv, n, k):
    import torch
    m = 512
    w, x, W, xd = _setup(qmv, n, k, m, seed=0)
    y = qmv.gemm(W, xd).cpu().numpy()
    torch.cuda.synchronize()
    xq, xs = oracle.quant_act(x)
    rng = np.random.default_rng(1)
    mm = np.concatenate([[0, m - 1, 0, m - 1], rng.integers(0, m, 252)])
    nn = np.concatenate([[0, 0, n - 1, n - 1], rng.integers(0, n, 252)])
    yr, b = oracle.q6k_gemm_pairs(oracle.Mat(oracle.Q6_K, n, k, w), xq, xs, mm, nn, nthreads=8)
    assert_parity(y[mm, nn][None, :], yr[None, :], b[None, :], f"gemm {n}x{k} sampled")
    # the exact int32 partials of a few sampled pairs, from the same MFMA path
    import torch as _t
    xq_d, _ = qmv.quant_act(xd)
    rows = slice(0, 64)
    p = qmv.partials(qweights(synth.FMT_Q6_K, 64, k, {kk: v[rows] for kk, v in w.items()}), xq_d[:40])
    _t.cuda.synchronize()
    mm2, nn2 = np.meshgrid(np.arange(40), np.arange(64), indexing="ij")
    _, i32 = oracle.q6k_partials(oracle.Mat(oracle.Q6_K, 64, k, {kk: v[rows] for kk, v in w.items()}), xq,
                                 mm2.ravel(), nn2.ravel())
    assert np.array_equal(p.cpu().numpy().reshape(-1, k // 32).astype(np.int64), i32)


def test_gemm_extreme_codes_and_scales(qmv):
    # w' = sc * (q - 32) at its extremes: sc = -128 with q = 0 gives +4096, sc = -128 with
    # q = 63 gives -3968, sc = 127 with q = 0 gives -4064; activations at +-127
    import torch
    n, k, m = 64, 512, 64
    w = synth.gen_weights(synth.FMT_Q6_K, n, k, seed=9)
    w["sc"][: n // 2] = -128
    w["sc"][n // 2:] = 127
    w["ql"][::2] = 0x00
    w["qh"][::2] = 0x00          # q = 0 on even rows
    w["ql"][1::2] = 0xFF
    w["qh"][1::2] = 0xFF         # q = 63 on odd rows
    x = np.sign(synth.gen_x(m, k, seed=9)).astype(np.float32) * np.float32(3.0)
    W = qweights(synth.FMT_Q6_K, n, k, w)
    xd = torch.from_numpy(x).cuda()
    xq, _ = qmv.quant_act(xd)
    p = qmv.partials(W, xq)
    y = qmv.gemm(W, xd)
    torch.cuda.synchronize()
    rq, _ = oracle.quant_act(x)
    om = oracle.Mat(oracle.Q6_K, n, k, w)
    mm, nn = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    _, i32 = oracle.q6k_partials(om, rq, mm.ravel(), nn.ravel())
    assert np.array_equal(p.cpu().numpy().reshape(m * n, k // 32).astype(np.int64), i32)
    yr, b, _, _ = oracle.q6k_gemm(om, x)
    assert_parity(y.cpu().numpy(), yr, b, "extreme gemm")


def test_gemm_all_codes_32_give_zero(qmv):
    import torch
    n, k, m = 64, 512, 33
    w = synth.gen_weights(synth.FMT_Q6_K, n, k, seed=4)
    w["ql"][:] = 0x00
    w["qh"][:] = 0xAA
    y = qmv.gemm(qweights(synth.FMT_Q6_K, n, k, w), torch.from_numpy(synth.gen_x(m, k, seed=4)).cuda())
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0.0)
