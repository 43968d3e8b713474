"""GPU parity of the routed-expert FFN over 4-bit codebook experts, through the C ABI.

For each routed expert e: h = SiLU(G_e x) * (U_e x), y = D_e h.  Each stage is checked
on its own input: h against the oracle's double h with a bound propagated from the
GEMV bound (|dSiLU/dz| <= 1.1), y against the oracle's GEMV of D_e applied to the
GPU's own h.  Invalid expert ids must give NaN rows.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import REL_TOL, assert_parity, x_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qmv():
    import torch
    assert torch.cuda.is_available()
    import bit_weight_quantized_dequant_amd as q
    q.lib()
    return q


def stacked_planes(n_experts, routed, n, k, matrix, seed):
    """Device planes [E][...] for n x k CB4 matrices; only the routed experts are filled."""
    import torch
    idx = torch.zeros((n_experts, n, k // 2), dtype=torch.uint8, device="cuda")
    cb = torch.zeros((n_experts, n, k // 128, 16), dtype=torch.float16, device="cuda")
    host = {}
    for e in routed:
        w = synth.gen_weights(synth.FMT_CB4, n, k, seed=seed, expert=e, matrix=matrix)
        idx[e] = torch.from_numpy(w["idx"]).cuda()
        cb[e] = torch.from_numpy(w["cb"].view(np.uint16).copy()).view(torch.float16).cuda()
        host[e] = w
    return {"idx": idx, "cb": cb}, host


def h_bound(g, u, bg, bu):
    """Bound on |h_gpu - h| from |g_gpu - g| <= tol*bg and |u_gpu - u| <= tol*bu."""
    eg, eu = REL_TOL * bg, REL_TOL * bu
    sg = g / (1 + np.exp(-g))
    return 1.1 * eg * (np.abs(u) + eu) + np.abs(sg) * eu + 1e-6 * np.abs(sg * u) + 1e-30


def run_moe(qmv, n_experts, dm, dff, ids, seed, rows_h=None, rows_y=None, expect="moe.cb4.gateup-silu+down2"):
    import torch
    routed = sorted({int(i) for i in ids if 0 <= i < n_experts})
    gp, gh = stacked_planes(n_experts, routed, dff, dm, 0, seed)
    up, uh = stacked_planes(n_experts, routed, dff, dm, 1, seed)
    dp, dh = stacked_planes(n_experts, routed, dm, dff, 2, seed)
    G = qmv.QWeights(qmv.CB4, dff, dm, gp)
    U = qmv.QWeights(qmv.CB4, dff, dm, up)
    D = qmv.QWeights(qmv.CB4, dm, dff, dp)
    x = synth.gen_x(1, dm, synth.DT_BF16, seed=seed)
    ids_t = torch.tensor(np.asarray(ids, dtype=np.int32), device="cuda")
    print(f"moe E={n_experts} dm={dm} dff={dff} ids={list(ids)}", flush=True)
    h, y = qmv.moe_ffn(G, U, D, n_experts, ids_t, x_to_device(x[0], synth.DT_BF16))
    torch.cuda.synchronize()
    assert qmv.last_path() == expect
    h, y = h.cpu().numpy(), y.cpu().numpy()
    for j, e in enumerate(ids):
        if not 0 <= e < n_experts:
            assert np.all(np.isnan(h[j])) and np.all(np.isnan(y[j]))
            continue
        gm = oracle.Mat(oracle.CB4, dff, dm, gh[e])
        um = oracle.Mat(oracle.CB4, dff, dm, uh[e])
        hr, g, u, bg, bu = oracle.moe_gateup(gm, um, x, oracle.BF16, rows=rows_h, nthreads=oracle.max_threads())
        hj = h[j] if rows_h is None else h[j][rows_h]
        err = np.abs(hj - hr)
        lim = h_bound(g, u, bg, bu)
        assert np.all(np.isfinite(hj)) and np.all(err <= lim), (j, e, float(np.max(err / lim)))
        dmat = oracle.Mat(oracle.CB4, dm, dff, dh[e])
        yr, by = oracle.gemv(dmat, h[j][None, :].astype(np.float32), oracle.F32, rows=rows_y, nthreads=oracle.max_threads())
        yj = y[j] if rows_y is None else y[j][rows_y]
        assert_parity(yj[None, :], yr, by, f"down expert {e}")


@pytest.mark.parametrize("force", ["", "moe.down1"])
def test_moe_small_with_invalid_id(qmv, monkeypatch, force):
    # the down stage with two rows per wave (default) and one (override)
    monkeypatch.setenv("QMV_FORCE_PATH", force)
    run_moe(qmv, n_experts=6, dm=512, dff=256, ids=[3, 0, 5, -1, 6], seed=1,
            expect="moe.cb4.gateup-silu+down" + ("" if force else "2"))


@pytest.mark.parametrize("force", ["", "moe.down1"])
def test_moe_ragged_sizes(qmv, monkeypatch, force):
    monkeypatch.setenv("QMV_FORCE_PATH", force)
    run_moe(qmv, n_experts=3, dm=1152, dff=640, ids=[2, 1], seed=2,
            expect="moe.cb4.gateup-silu+down" + ("" if force else "2"))


def test_moe_deepseek_like_layer_top8_of_256(qmv):
    # 256 experts of gate/up 2048 x 7168 and down 7168 x 2048; top-8 ids for token 0
    # (every row of h and y of each routed expert is checked)
    ids = synth.gen_moe_ids(1, 256, 8, seed=0)[0]
    run_moe(qmv, n_experts=256, dm=7168, dff=2048, ids=ids, seed=0)
