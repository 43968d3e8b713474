"""GPU parity of the q6_K prefill GEMM (int8 MFMA) against the CPU oracle.

Bar: the int32 per-block partials I32[m][n][c] are bit-exact; every output is within
2e-3 * sum_k |w| |x_hat| of the oracle's double result (x_hat = xs * xq, the quantized
activations, as the oracle defines the GEMM); full workload sizes are checked on every
output of a dozen token rows and every token of several weight rows (the oracle computes
those pairs one by one; the whole product would take it minutes).
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


def gemm_check_pairs(m, n, seed=1):
    """(m, n) pairs for a full-size GEMM: every output of 12 token rows (the first, the
    last, the two around each 128-token tile edge and 4 random ones) and every token of 8
    weight rows (the first, the last, the two around the 64-row tile edge and 4 random
    ones); the full product would take the oracle minutes."""
    rng = np.random.default_rng(seed)
    toks = sorted({0, m - 1, 127 % m, 128 % m, 255 % m, 256 % m, *rng.integers(0, m, 4).tolist()})
    rows = sorted({0, n - 1, 63 % n, 64 % n, *rng.integers(0, n, 4).tolist()})
    a = np.meshgrid(np.array(toks), np.arange(n), indexing="ij")
    b = np.meshgrid(np.arange(m), np.array(rows), indexing="ij")
    return np.concatenate([a[0].ravel(), b[0].ravel()]), np.concatenate([a[1].ravel(), b[1].ravel()])


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
    mm, nn = gemm_check_pairs(m, n)
    yr, b = oracle.q6k_gemm_pairs(oracle.Mat(oracle.Q6_K, n, k, w), xq, xs, mm, nn, nthreads=oracle.max_threads())
    assert_parity(y[mm, nn][None, :], yr[None, :], b[None, :], f"gemm {n}x{k} rows and columns")
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


# ------------------------------------------------------- pre-expanded planes

def test_plane_holds_the_exact_hi_lo_split(qmv):
    # 64 H + L == sc * (q - 32) for every weight, H in [-64, 64], L in [0, 63]; q from the
    # oracle's integer decode, sc with both signs and both extremes
    import torch
    n, k = 37, 1024
    w = synth.gen_weights(synth.FMT_Q6_K, n, k, seed=3)
    w["sc"][::3] = -w["sc"][::3]
    w["sc"][1, 0, :] = -128
    w["sc"][2, 0, :] = 127
    W = qweights(synth.FMT_Q6_K, n, k, w)
    try:
        plane = qmv.register_plane(W)
        torch.cuda.synchronize()
        assert qmv.last_path() == "plane.q6k.expand"
        p = plane.cpu().numpy().view(np.int8).astype(np.int64)
    finally:
        qmv.unregister_plane(W)
    # [row group][32-block][H, L][lane][16]: lane l holds row 32 g + l % 32, k 32 c + 16 (l / 32) ..
    G = -(-n // 32)
    assert p.size == 2 * 32 * G * k
    f = p.reshape(G, k // 32, 2, 2, 32, 16)            # [g][c][H/L][l // 32][l % 32][16]
    f = f.transpose(2, 0, 4, 1, 3, 5).reshape(2, G * 32, k)
    H, L = f[0][:n], f[1][:n]
    assert not f[:, n:].any()
    q = oracle.codes(oracle.Mat(oracle.Q6_K, n, k, w)).astype(np.int64)
    sc = np.repeat(w["sc"].reshape(n, k // 16).astype(np.int64), 16, axis=1)
    assert np.array_equal(64 * H + L, sc * (q - 32))
    assert L.min() >= 0 and L.max() <= 63 and H.min() >= -64 and H.max() <= 64


@pytest.mark.parametrize("n,k,m", [(64, 512, 128), (70, 768, 45), (257, 2048, 130), (4096, 1024, 512), (3, 256, 1),
                                   (8192, 256, 512)])
@pytest.mark.parametrize("force", ["", "gemm.ks1", "gemm.ks2"])
def test_gemm_with_plane_is_byte_identical(qmv, monkeypatch, n, k, m, force):
    # outputs and int32 partials with the plane equal those of the in-kernel expansion bit
    # for bit (the expansion is an integer transform), with four-wave workgroups and with
    # eight-wave K-split ones (forced either way on every shape); the partials also equal the
    # oracle's
    import torch
    monkeypatch.setenv("QMV_FORCE_PATH", force)
    w, x, W, xd = _setup(qmv, n, k, m, seed=n + 7 * m)
    xq, xs = qmv.quant_act(xd)
    y0 = qmv.gemm_q8(W, xq, xs)
    assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.rowmajor-act"
    p0 = qmv.partials(W, xq)
    qmv.register_plane(W)
    try:
        y1 = qmv.gemm_q8(W, xq, xs)
        assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.rowmajor-act.plane"
        p1 = qmv.partials(W, xq)
        assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.partials.plane"
        y2 = qmv.gemm(W, xd)
        assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.plane"
    finally:
        qmv.unregister_plane(W)
    y3 = qmv.gemm_q8(W, xq, xs)
    assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.rowmajor-act"
    torch.cuda.synchronize()
    y0, y1, y2, y3 = (t.cpu().numpy().view(np.int32) for t in (y0, y1, y2, y3))
    assert np.array_equal(y0, y1) and np.array_equal(y0, y2) and np.array_equal(y0, y3)
    assert np.array_equal(p0.cpu().numpy(), p1.cpu().numpy())
    if n * m <= 64 * 130:
        rq, _ = oracle.quant_act(x)
        mm, nn = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        _, i32 = oracle.q6k_partials(oracle.Mat(oracle.Q6_K, n, k, w), rq, mm.ravel(), nn.ravel())
        assert np.array_equal(p1.cpu().numpy().reshape(m * n, k // 32).astype(np.int64), i32)


def test_plane_labels_opt_out_and_fallback(qmv, monkeypatch):
    import torch
    n, k, m = 96, 512, 70
    w, x, W, xd = _setup(qmv, n, k, m, seed=5)
    xq, xs = qmv.quant_act(xd)
    ref = qmv.gemm_q8(W, xq, xs)
    # opted out: registration builds nothing, the GEMM names the reason
    monkeypatch.setenv("QMV_Q6K_EXP", "0")
    qmv.register_plane(W)
    assert qmv.last_path() == "plane.q6k(exp=off)"
    y_off = qmv.gemm_q8(W, xq, xs)
    assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.rowmajor-act(exp=off)"
    monkeypatch.delenv("QMV_Q6K_EXP")
    # registered for 96 rows; a descriptor over the same codes with 95 rows must not use it
    qmv.register_plane(W)
    try:
        W95 = qmv.QWeights(synth.FMT_Q6_K, n - 1, k, W.planes)
        y95 = qmv.gemm_q8(W95, xq, xs)
        assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.rowmajor-act(fallback!)"
        y_plane = qmv.gemm_q8(W, xq, xs)
        assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.rowmajor-act.plane"
    finally:
        qmv.unregister_plane(W)
    torch.cuda.synchronize()
    ref = ref.cpu().numpy()
    assert np.array_equal(y_off.cpu().numpy().view(np.int32), ref.view(np.int32))
    assert np.array_equal(y_plane.cpu().numpy().view(np.int32), ref.view(np.int32))
    assert np.array_equal(y95.cpu().numpy().view(np.int32), ref[:, : n - 1].copy().view(np.int32))


@pytest.mark.parametrize("n,k", [(11008, 4096), (4096, 11008)])
def test_gemm_prefill_shapes_with_plane(qmv, n, k):
    # the workload shapes: byte-identical with and without the plane, and within the bound
    # of the oracle on sampled pairs
    import torch
    m = 512
    w, x, W, xd = _setup(qmv, n, k, m, seed=0)
    y0 = qmv.gemm(W, xd)
    qmv.register_plane(W)
    try:
        y1 = qmv.gemm(W, xd)
        assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.plane"
    finally:
        qmv.unregister_plane(W)
    torch.cuda.synchronize()
    y0, y1 = y0.cpu().numpy(), y1.cpu().numpy()
    assert np.array_equal(y0.view(np.int32), y1.view(np.int32))
    xq, xs = oracle.quant_act(x)
    mm, nn = gemm_check_pairs(m, n, seed=2)
    yr, b = oracle.q6k_gemm_pairs(oracle.Mat(oracle.Q6_K, n, k, w), xq, xs, mm, nn, nthreads=oracle.max_threads())
    assert_parity(y1[mm, nn][None, :], yr[None, :], b[None, :], f"gemm plane {n}x{k} rows and columns")


def test_collected_weights_leave_no_stale_plane(qmv):
    # a registered matrix that is garbage-collected without unregister_plane drops the
    # library's record with it: a new matrix of the same shape whose tensors reuse the freed
    # addresses must run the in-kernel expansion, not the old plane
    import gc
    import torch
    n, k, m = 64, 512, 40
    w, x, W, xd = _setup(qmv, n, k, m, seed=11)
    xq, xs = qmv.quant_act(xd)
    qmv.register_plane(W)
    qmv.gemm_q8(W, xq, xs)
    assert qmv.last_path().endswith(".plane")
    addr = W.planes["ql"].data_ptr()
    del W
    gc.collect()
    torch.cuda.synchronize()
    w2 = synth.gen_weights(synth.FMT_Q6_K, n, k, seed=12)
    W2 = qweights(synth.FMT_Q6_K, n, k, w2)
    y = qmv.gemm_q8(W2, xq, xs)
    assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.rowmajor-act"
    torch.cuda.synchronize()
    yr, b = oracle.q6k_gemm_pairs(oracle.Mat(oracle.Q6_K, n, k, w2), *oracle.quant_act(x),
                                  *[a.ravel() for a in np.meshgrid(np.arange(m), np.arange(n), indexing="ij")])
    assert_parity(y.cpu().numpy().reshape(1, -1), yr[None, :], b[None, :], "gemm after a collected plane")
    print("codes address reused:", W2.planes["ql"].data_ptr() == addr)


def test_gemm_ws_reuses_the_quantized_activations(qmv):
    # one quantization serves a second matrix: gemm_ws on the workspace that gemm(W1, x) left
    # equals gemm(W2, x) bit for bit, with and without W2's plane; row-major activations
    # (gemm_q8) give the same bytes too
    import torch
    n, k, m = 200, 1024, 150
    w1, x, W1, xd = _setup(qmv, n, k, m, seed=21)
    w2 = synth.gen_weights(synth.FMT_Q6_K, n + 37, k, seed=22)
    W2 = qweights(synth.FMT_Q6_K, n + 37, k, w2)
    ws = torch.empty(qmv.workspace_bytes(W1, m), dtype=torch.uint8, device="cuda")
    qmv.gemm(W1, xd, ws=ws)
    y2 = qmv.gemm_ws(W2, ws, m=m)
    assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split"
    ref = qmv.gemm(W2, xd)
    xq, xs = qmv.quant_act(xd)
    y8 = qmv.gemm_q8(W2, xq, xs)
    qmv.register_plane(W2)
    try:
        y3 = qmv.gemm_ws(W2, ws, m=m)
        assert qmv.last_path() == "gemm.q6k.mfma-i8-32x32x32.hl-split.plane"
    finally:
        qmv.unregister_plane(W2)
    torch.cuda.synchronize()
    ref = ref.cpu().numpy().view(np.int32)
    for y in (y2, y3, y8):
        assert np.array_equal(y.cpu().numpy().view(np.int32), ref)
    yr, b, _, _ = oracle.q6k_gemm(oracle.Mat(oracle.Q6_K, n + 37, k, w2), x, nthreads=oracle.max_threads())
    assert_parity(y2.cpu().numpy(), yr, b, "gemm_ws")
