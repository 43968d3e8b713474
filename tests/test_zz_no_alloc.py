"""The no-allocation q6_K GEMM (qmm_gemm_noalloc) against qmm_gemm, through the C ABI.

The two run the same kernels; the no-allocation form quantizes into the library's own
per-GPU scratch array instead of a caller workspace, so its output must equal qmm_gemm's
bit for bit.  Two calls in a row, the second on a smaller input, check that the array's
address and the carry-over of the first call's contents do not matter.
"""
import ctypes as C

import numpy as np
import pytest

import synth
from helpers import qweights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qmv():
    import torch
    assert torch.cuda.is_available()
    import bit_weight_quantized_dequant_amd as q
    q.lib()
    return q


def _case(qmv, n, k, m, seed):
    import torch
    w = synth.gen_weights(synth.FMT_Q6_K, n, k, seed=seed)
    W = qweights(synth.FMT_Q6_K, n, k, w)
    x = torch.from_numpy(synth.gen_x(m, k, seed=seed)).cuda()
    return W, x


def test_noalloc_gemm_equals_workspace_gemm_on_two_calls(qmv):
    import torch
    L = qmv.lib()
    stream = torch.cuda.current_stream().cuda_stream
    results = []
    for n, k, m, seed in [(4096, 11008, 512, 1), (300, 2048, 77, 2)]:
        print(f"noalloc case n={n} k={k} m={m}", flush=True)
        W, x = _case(qmv, n, k, m, seed)
        y_ref = torch.empty((m, n), dtype=torch.float32, device="cuda")
        ws = torch.empty(qmv.workspace_bytes(W, m), dtype=torch.uint8, device="cuda")
        assert L.qmm_gemm(W.ref, m, x.data_ptr(), y_ref.data_ptr(), ws.data_ptr(), ws.numel(), C.c_void_p(stream)) == 0
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        assert L.qmm_gemm_noalloc(W.ref, m, x.data_ptr(), y.data_ptr(), C.c_void_p(stream)) == 0
        assert qmv.last_path().startswith("gemm.q6k.")
        results.append((y_ref, y))
    torch.cuda.synchronize()
    for y_ref, y in results:
        a, b = y_ref.cpu().numpy(), y.cpu().numpy()
        assert np.all(np.isfinite(b))
        assert np.array_equal(a.view(np.int32), b.view(np.int32))


def test_noalloc_gemm_binding_and_limit(qmv):
    import torch
    W, x = _case(qmv, 64, 512, 40, 3)
    y = torch.empty((40, 64), dtype=torch.float32, device="cuda")
    qmv.gemm_noalloc(W, x, y)
    ref = qmv.gemm(W, x)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.int32), ref.cpu().numpy().view(np.int32))
    big = qweights(synth.FMT_Q6_K, 8, 29184, synth.gen_weights(synth.FMT_Q6_K, 8, 29184, seed=4))
    with pytest.raises(qmv.QmvError):
        qmv.gemm_noalloc(big, torch.zeros((512, 29184), dtype=torch.float32, device="cuda"),
                         torch.empty((512, 8), dtype=torch.float32, device="cuda"))
