"""GPU parity of the decode GEMVs against the CPU oracle, through the C ABI.

Bar: every output within 2e-3 * sum_k |w||x| of the oracle's double result;
x = e_j returns column j of W bit-exactly; outputs are deterministic and
row-permutation equivariant bit-for-bit.  Full workload sizes are checked on
sampled rows (the oracle computes those rows one by one).
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


def run_case(qmv, fmt, n, k, m, xt, seed, rows=None, expect_path=None):
    import torch
    w = synth.gen_weights(fmt, n, k, seed=seed)
    x = synth.gen_x(m, k, xt, seed=seed)
    print(f"case fmt={fmt} n={n} k={k} m={m} xt={xt} seed={seed}", flush=True)
    W = qweights(fmt, n, k, w)
    y = qmv.gemv(W, x_to_device(x, xt))
    torch.cuda.synchronize()
    if expect_path:
        assert qmv.last_path() == expect_path
    y = y.cpu().numpy()
    om = oracle.Mat(fmt, n, k, w)
    if rows is None:
        yr, b = oracle.gemv(om, x, xt)
        return assert_parity(y, yr, b, f"fmt={fmt} {n}x{k} m={m}")
    yr, b = oracle.gemv(om, x, xt, rows=rows)
    return assert_parity(y[:, rows], yr, b, f"fmt={fmt} {n}x{k} m={m} sampled")


def sample_rows(n, count=96, seed=0):
    rng = np.random.default_rng(seed)
    r = set(rng.choice(n, size=min(n, count), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(r), dtype=np.int64)


# ------------------------------------------------------------------ q4_0

Q4_SMALL = [(1, 32), (7, 64), (64, 2048 + 160), (130, 4096), (33, 11008), (300, 2048 * 8)]


@pytest.mark.parametrize("n,k", Q4_SMALL)
@pytest.mark.parametrize("path", ["default", "q4_0.cvt"])
def test_q4_0_small_full_parity(qmv, monkeypatch, n, k, path):
    if path != "default":
        monkeypatch.setenv("QMV_FORCE_PATH", path)
    expect = "q4_0.lds-x.cvt-ubyte" if path == "q4_0.cvt" else "q4_0.lds-x.fma-mix"
    run_case(qmv, synth.FMT_Q4_0, n, k, 1, synth.DT_F32, seed=n + k, expect_path=expect)


@pytest.mark.parametrize("m", [2, 3, 4, 8])
@pytest.mark.parametrize("xt", [synth.DT_F32, synth.DT_BF16])
def test_q4_0_batched(qmv, m, xt):
    run_case(qmv, synth.FMT_Q4_0, 96, 2048, m, xt, seed=m)


@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_q4_0_full_size_sampled(qmv, n, k):
    run_case(qmv, synth.FMT_Q4_0, n, k, 1, synth.DT_F32, seed=0, rows=sample_rows(n))


def test_q4_0_unit_vector_returns_column_exactly(qmv):
    import torch
    n, k = 200, 4096
    w = synth.gen_weights(synth.FMT_Q4_0, n, k, seed=5)
    W = qweights(synth.FMT_Q4_0, n, k, w)
    dense = oracle.dequant(oracle.Mat(synth.FMT_Q4_0, n, k, w)).astype(np.float32)
    for j in (0, 1, 16, 31, 2047, 4095):
        e = np.zeros((1, k), dtype=np.float32)
        e[0, j] = 1.0
        y = qmv.gemv(W, x_to_device(e, synth.DT_F32))
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy()[0], dense[:, j]), j


def test_q4_0_deterministic_and_permutation_equivariant(qmv):
    import torch
    n, k = 512, 4096
    w = synth.gen_weights(synth.FMT_Q4_0, n, k, seed=9)
    x = x_to_device(synth.gen_x(1, k, seed=9), synth.DT_F32)
    W = qweights(synth.FMT_Q4_0, n, k, w)
    y1 = qmv.gemv(W, x).cpu().numpy()
    y2 = qmv.gemv(W, x).cpu().numpy()
    assert np.array_equal(y1, y2)
    perm = np.random.default_rng(1).permutation(n)
    Wp = qweights(synth.FMT_Q4_0, n, k, {"qs": w["qs"][perm], "d": w["d"][perm]})
    yp = qmv.gemv(Wp, x).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(yp[0], y1[0, perm])


def test_q4_0_limit_is_reported(qmv):
    import torch
    W = qweights(synth.FMT_Q4_0, 4, 2048 * 9, synth.gen_weights(synth.FMT_Q4_0, 4, 2048 * 9))
    x = torch.zeros((1, 2048 * 9), dtype=torch.float32, device="cuda")
    with pytest.raises(qmv.QmvError) as e:
        qmv.gemv(W, x)
    assert e.value.code == -9
