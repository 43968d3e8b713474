"""GPU parity of the GEMVs over per-32 int8 activations (qmv_gemv_q8), through the C ABI.

The oracle forms the exact integer block sums in double: for q4_0, I = sum (q - 8) * xq and
y = sum d * xs * I; for q6_K, the q6_K contraction's sum_s d * sum_c xs * sum_j sc * sum
(q - 32) * xq.  The bar is |y_gpu - y_ref| <= 2e-3 * sum |w| |xs * xq| per element.  The activations
come from the oracle's quantizer (or from the GPU quantizer, checked bit-exact against it).
Full workload sizes are checked on sampled rows.
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
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_weight_quantized_dequant_amd as q
    q.lib()
    return q


def q8_path(m, k, fmt=synth.FMT_Q4_0):
    return "q4_0.q8.lds-x.dot4" if fmt == synth.FMT_Q4_0 else "q6_K.q8.lds-x.dot4"


def run_q8(qmv, n, k, m, seed, rows=None, expect=None, gpu_quant=False, x=None, fmt=synth.FMT_Q4_0):
    import torch
    print(f"case q8 fmt={fmt} n={n} k={k} m={m} seed={seed} gpu_quant={gpu_quant}", flush=True)
    w = synth.gen_weights(fmt, n, k, seed=seed)
    if x is None:
        x = synth.gen_x(m, k, synth.DT_F32, seed=seed)
    xq, xs = oracle.quant_act(x)
    W = qweights(fmt, n, k, w)
    if gpu_quant:
        xq_d, xs_d = qmv.quant_act(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(xq_d.cpu().numpy(), xq) and np.array_equal(xs_d.cpu().numpy(), xs)
    else:
        xq_d, xs_d = torch.from_numpy(xq).cuda(), torch.from_numpy(xs).cuda()
    y = qmv.gemv_q8(W, xq_d, xs_d)
    torch.cuda.synchronize()
    if expect:
        assert qmv.last_path() == expect
    y = y.cpu().numpy()
    om = oracle.Mat(fmt, n, k, w)
    rr = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    if fmt == synth.FMT_Q4_0:
        yr, b = oracle.q4_0_gemv_q8(om, xq, xs, rows=rr, nthreads=oracle.max_threads())
    else:
        mm, nn = np.meshgrid(np.arange(m), rr, indexing="ij")
        yr, b = oracle.q6k_gemm_pairs(om, xq, xs, mm.ravel(), nn.ravel(), nthreads=oracle.max_threads())
        yr, b = yr.reshape(m, len(rr)), b.reshape(m, len(rr))
    return assert_parity(y[:, rr], yr, b, f"q8 fmt={fmt} {n}x{k} m={m}")


@pytest.mark.parametrize("n,k", [(1, 32), (7, 64), (64, 2048 + 160), (130, 4096), (33, 11008), (300, 2048 * 8)])
def test_q8_small_full_parity(qmv, n, k):
    run_q8(qmv, n, k, 1, seed=n + k, expect=q8_path(1, k))


@pytest.mark.parametrize("m", [2, 3, 4, 8])
@pytest.mark.parametrize("n,k", [(97, 2048), (41, 4096 + 64), (9, 11008)])
def test_q8_batched(qmv, n, k, m):
    run_q8(qmv, n, k, m, seed=m * 7 + k, expect=q8_path(m, k))


@pytest.mark.parametrize("n,k,m", [(5, 4096, 1), (9, 4096 + 64, 1), (3, 32 * 65, 2), (2, 16384, 1)])
def test_q8_row_and_block_tails(qmv, n, k, m):
    # row counts that leave part of the last workgroup idle, a ragged last block column
    run_q8(qmv, n, k, m, seed=n * k + m, expect=q8_path(m, k))


@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_q8_full_size_sampled(qmv, n, k, m):
    # the decode shapes, with the GPU quantizer in front (checked bit-exact)
    run_q8(qmv, n, k, m, seed=m, rows=np.array(sorted({0, n - 1} | set(range(1, n, 97)))),
           expect=q8_path(m, k), gpu_quant=True)


def test_q8_special_activations(qmv):
    # zero blocks (xs = 0, xq = 0), a block of one huge value, exact-integer blocks
    k = 4096
    x = synth.gen_x(2, k, synth.DT_F32, seed=3)
    x[0, :64] = 0.0
    x[1, 32:64] = 0.0
    x[1, 64] = 1e30
    x[0, 128:160] = np.arange(-16, 16, dtype=np.float32) * 8
    run_q8(qmv, 65, k, 2, seed=3, x=x, gpu_quant=True)


def test_q8_deterministic_and_permutation_equivariant(qmv):
    import torch
    n, k = 512, 4096
    w = synth.gen_weights(synth.FMT_Q4_0, n, k, seed=9)
    xq, xs = oracle.quant_act(synth.gen_x(1, k, seed=9))
    xq_d, xs_d = torch.from_numpy(xq).cuda(), torch.from_numpy(xs).cuda()
    W = qweights(synth.FMT_Q4_0, n, k, w)
    y1 = qmv.gemv_q8(W, xq_d, xs_d).cpu().numpy()
    y2 = qmv.gemv_q8(W, xq_d, xs_d).cpu().numpy()
    assert np.array_equal(y1, y2)
    perm = np.random.default_rng(1).permutation(n)
    Wp = qweights(synth.FMT_Q4_0, n, k, {"qs": w["qs"][perm], "d": w["d"][perm]})
    yp = qmv.gemv_q8(Wp, xq_d, xs_d).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(yp[0], y1[0, perm])


def test_q8_limits(qmv):
    import torch
    # k beyond 16384, and staged activations beyond one workgroup's LDS, are refused
    for n, k, m in [(4, 16384 + 32, 1), (4, 16384, 8)]:
        W = qweights(synth.FMT_Q4_0, n, k, synth.gen_weights(synth.FMT_Q4_0, n, k, seed=1))
        xq = torch.zeros((m, k), dtype=torch.int8, device="cuda")
        xs = torch.zeros((m, k // 32), dtype=torch.float32, device="cuda")
        with pytest.raises(qmv.QmvError) as e:
            qmv.gemv_q8(W, xq, xs)
        assert e.value.code == -9


# ------------------------------------------------------------------ q6_K

@pytest.mark.parametrize("n,k", [(1, 256), (7, 512), (64, 2048 + 256), (130, 4096), (33, 11008), (300, 16384)])
def test_q6k_q8_small_full_parity(qmv, n, k):
    run_q8(qmv, n, k, 1, seed=n + k, expect=q8_path(1, k, synth.FMT_Q6_K), fmt=synth.FMT_Q6_K)


@pytest.mark.parametrize("m", [2, 3, 4, 8])
@pytest.mark.parametrize("n,k", [(97, 2048), (41, 4096 + 256), (9, 11008)])
def test_q6k_q8_batched(qmv, n, k, m):
    # covers the rolled unit loop (batch rows x units per lane above 8) and the unrolled one
    run_q8(qmv, n, k, m, seed=m * 7 + k, expect=q8_path(m, k, synth.FMT_Q6_K), fmt=synth.FMT_Q6_K)


@pytest.mark.parametrize("n,k,m", [(5, 4096, 1), (9, 4096 + 256, 1), (3, 256 * 5, 2), (2, 16384, 1)])
def test_q6k_q8_row_and_unit_tails(qmv, n, k, m):
    run_q8(qmv, n, k, m, seed=n * k + m, expect=q8_path(m, k, synth.FMT_Q6_K), fmt=synth.FMT_Q6_K)


@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_q6k_q8_full_size_sampled(qmv, n, k, m):
    run_q8(qmv, n, k, m, seed=m, rows=np.array(sorted({0, n - 1} | set(range(1, n, 97)))),
           expect=q8_path(m, k, synth.FMT_Q6_K), gpu_quant=True, fmt=synth.FMT_Q6_K)


def test_q6k_q8_special_activations(qmv):
    k = 4096
    x = synth.gen_x(2, k, synth.DT_F32, seed=4)
    x[0, :64] = 0.0
    x[1, 32:64] = 0.0
    x[1, 64] = -1e30
    x[0, 256:288] = np.arange(-16, 16, dtype=np.float32) * 8
    run_q8(qmv, 65, k, 2, seed=4, x=x, gpu_quant=True, fmt=synth.FMT_Q6_K)


def test_q6k_q8_limits(qmv):
    import torch
    for n, k, m in [(4, 16384 + 256, 1), (4, 16384, 8)]:
        W = qweights(synth.FMT_Q6_K, n, k, synth.gen_weights(synth.FMT_Q6_K, n, k, seed=1))
        xq = torch.zeros((m, k), dtype=torch.int8, device="cuda")
        xs = torch.zeros((m, k // 32), dtype=torch.float32, device="cuda")
        with pytest.raises(qmv.QmvError) as e:
            qmv.gemv_q8(W, xq, xs)
        assert e.value.code == -9
