"""GPU checks of the unpack stage (dense dequantization) and of the int8 activation
quantizer, both against the CPU oracle: bit-exact where the values are exact."""
import numpy as np
import pytest

import oracle
import synth
from helpers import qweights
from test_oracle import load_golden

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qmv():
    import torch
    assert torch.cuda.is_available()
    import bit_weight_quantized_dequant_amd as q
    q.lib()
    return q


@pytest.mark.parametrize("fmt,n,k", [(synth.FMT_Q4_0, 33, 4096), (synth.FMT_Q6_K, 17, 2048),
                                     (synth.FMT_CB4, 19, 1024), (synth.FMT_Q6_K, 256, 1024),
                                     (synth.FMT_CB8, 21, 640)])
def test_dequant_bit_exact(qmv, fmt, n, k):
    import torch
    w = synth.gen_weights(fmt, n, k, seed=n)
    out = qmv.dequant(qweights(fmt, n, k, w))
    torch.cuda.synchronize()
    assert qmv.last_path().startswith("dequant.")
    ref = oracle.dequant(oracle.Mat(fmt, n, k, w))
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)
    if fmt in (synth.FMT_Q4_0, synth.FMT_Q6_K):
        codes = oracle.codes(oracle.Mat(fmt, n, k, w))
        assert codes.min() >= 0 and codes.max() <= (15 if fmt == synth.FMT_Q4_0 else 63)


def test_dequant_aq_within_two_roundings(qmv):
    import torch
    n, k = 23, 512
    w = synth.gen_weights(synth.FMT_AQ2X8, n, k, seed=4)
    out = qmv.dequant(qweights(synth.FMT_AQ2X8, n, k, w)).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    ref = oracle.dequant(oracle.Mat(synth.FMT_AQ2X8, n, k, w))
    # s*(C1+C2): one rounding of the sum, one of the product (each <= 2^-24 relative)
    s = w["s"].astype(np.float64)[:, None]
    mag = s * (np.abs(w["cbk"][0][w["codes"][:, :, 0]].astype(np.float64)) +
               np.abs(w["cbk"][1][w["codes"][:, :, 1]].astype(np.float64))).reshape(n, k)
    assert np.all(np.abs(out - ref) <= 2.0 ** -23 * (mag + np.abs(ref)))


def test_dequant_aq3_within_three_roundings(qmv):
    import torch
    n, k = 23, 512
    w = synth.gen_weights(synth.FMT_AQ3X8, n, k, seed=4)
    out = qmv.dequant(qweights(synth.FMT_AQ3X8, n, k, w)).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    assert qmv.last_path() == "dequant.aq3x8"
    ref = oracle.dequant(oracle.Mat(synth.FMT_AQ3X8, n, k, w))
    # s*((C1+C2)+C3): two roundings of the sums, one of the product (each <= 2^-24 relative)
    s = w["s"].astype(np.float64)[:, None]
    mag = s * sum(np.abs(w["cbk"][b][w["codes"][:, :, b]].astype(np.float64)) for b in range(3)).reshape(n, k)
    assert np.all(np.abs(out - ref) <= 3 * 2.0 ** -24 * (mag + np.abs(ref)))


def _quant_gpu(qmv, x):
    import torch
    xq, xs = qmv.quant_act(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert qmv.last_path() == "quant_act.dpp8"
    return xq.cpu().numpy(), xs.cpu().numpy()


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (512, 4096), (512, 11008)])
def test_quantizer_bit_exact_random(qmv, m, k):
    x = synth.gen_x(m, k, seed=m + k)
    xq, xs = _quant_gpu(qmv, x)
    rq, rs = oracle.quant_act(x)
    assert np.array_equal(xq, rq)
    assert np.array_equal(xs.view(np.uint32), rs.view(np.uint32))


def test_quantizer_golden_and_edge_blocks(qmv):
    g = load_golden("quant_act.txt")
    rng = np.random.default_rng(5)
    blocks = [np.array(g["a_x"], dtype=np.float32), np.zeros(32, np.float32),
              np.array(g["c_x"], dtype=np.float32),
              # ties after division: x = (j + 0.5) * xs for a power-of-two amax
              (np.arange(32, dtype=np.float32) - 15.5) * np.float32(2.0) ** -3,
              # tiny and huge magnitudes, a single nonzero, negative maximum
              rng.standard_normal(32).astype(np.float32) * np.float32(1e-30),
              rng.standard_normal(32).astype(np.float32) * np.float32(1e30),
              np.eye(32, dtype=np.float32)[7] * np.float32(-3.0)]
    x = np.concatenate(blocks)[None, :]
    xq, xs = _quant_gpu(qmv, x)
    rq, rs = oracle.quant_act(x)
    assert np.array_equal(xq, rq)
    assert np.array_equal(xs.view(np.uint32), rs.view(np.uint32))
    assert xq[0, :32].tolist() == g["a_xq"] and xq[0, 64:96].tolist() == g["c_xq"]


def test_library_loaded_before_torch(qmv):
    # torch carries its own HIP runtime; the binding imports torch before it opens the library,
    # so a program that loads the library first still runs one runtime (checked in a fresh
    # process, since this one has imported torch already)
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    code = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import bit_weight_quantized_dequant_amd as q\n"
        "q.lib()\n"
        "import torch, numpy as np, synth, oracle\n"
        "x = synth.gen_x(2, 256, seed=3)\n"
        "xq, xs = q.quant_act(torch.from_numpy(x).cuda())\n"
        "torch.cuda.synchronize()\n"
        "oq, os_ = oracle.quant_act(x)\n"
        "assert np.array_equal(xq.cpu().numpy(), oq) and np.array_equal(xs.cpu().numpy(), os_)\n"
        "print('ok')\n" % (os.path.dirname(here), here))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=100)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_read_ceiling_reads_and_writes_nothing(qmv):
    # the measurement kernel leaves its sink alone for ordinary data (the XOR of a zero
    # buffer is 0, not the sentinel), and covers ragged sizes
    import torch
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    for nbytes in (16, 4096 * 16 + 48, 25362432):
        buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        qmv.read_ceiling(buf, sink)
        torch.cuda.synchronize()
        assert qmv.last_path() == "read-ceiling.16B-per-thread"
        assert sink.item() == 7
