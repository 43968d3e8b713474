"""GPU parity of the decode GEMVs against the CPU oracle, through the C ABI.

Bar: every output within 2e-3 * sum_k |w||x| of the oracle's double result;
x = e_j returns column j of W bit-exactly; outputs are deterministic and
row-permutation equivariant bit-for-bit.  Full workload sizes are checked on every
output row (the oracle runs multithreaded over rows).
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
        yr, b = oracle.gemv(om, x, xt, nthreads=oracle.max_threads())
        return assert_parity(y, yr, b, f"fmt={fmt} {n}x{k} m={m}")
    yr, b = oracle.gemv(om, x, xt, rows=rows, nthreads=oracle.max_threads())
    return assert_parity(y[:, rows], yr, b, f"fmt={fmt} {n}x{k} m={m} sampled")


# ------------------------------------------------------------------ q4_0

Q4_SMALL = [(1, 32), (7, 64), (64, 2048 + 160), (130, 4096), (33, 11008), (300, 2048 * 8)]


def q4_path(m, k, n=1):
    # batches and rows longer than 16384 go through the K-chunked kernel; batch 1 through the
    # one-shot kernel, two rows per wave while the blocks per lane are at most 4 and the
    # matrix has at most 32 rows per CU
    import torch
    bpl = -(-(k // 32) // 64)
    if bpl > 8 or m > 1:
        # from three batch rows up the weights are expanded to fp32 once per block
        return "q4_0.lds-x-chunked.fmac" if m >= 3 else "q4_0.lds-x-chunked.fma-mix"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return "q4_0.lds-x.fma-mix.2row" if bpl <= 4 and n <= 32 * cus else "q4_0.lds-x.fma-mix"


@pytest.mark.parametrize("n,k", Q4_SMALL)
@pytest.mark.parametrize("path", ["default", "q4_0.r1", "q4_0.cvt", "q4_0.chunked"])
def test_q4_0_small_full_parity(qmv, monkeypatch, n, k, path):
    if path != "default":
        monkeypatch.setenv("QMV_FORCE_PATH", path)
    expect = {"default": q4_path(1, k), "q4_0.r1": "q4_0.lds-x.fma-mix", "q4_0.cvt": "q4_0.lds-x.cvt-ubyte",
              "q4_0.chunked": "q4_0.lds-x-chunked.fma-mix"}[path]
    run_case(qmv, synth.FMT_Q4_0, n, k, 1, synth.DT_F32, seed=n + k, expect_path=expect)


@pytest.mark.parametrize("m", [2, 3, 4, 8])
@pytest.mark.parametrize("xt", [synth.DT_F32, synth.DT_BF16])
def test_q4_0_batched(qmv, m, xt):
    run_case(qmv, synth.FMT_Q4_0, 97, 2048, m, xt, seed=m, expect_path=q4_path(m, 2048))


@pytest.mark.parametrize("n,k,m", [(5, 4096, 2), (9, 4096 + 64, 1), (33, 8192, 1), (2, 2048 * 3, 1)])
def test_q4_0_two_rows_per_wave_tails(qmv, n, k, m):
    # odd row counts (the last wave's second row is past the end), ragged block tails
    run_case(qmv, synth.FMT_Q4_0, n, k, m, synth.DT_F32, seed=n * k + m, expect_path=q4_path(m, k))


@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_q4_0_full_size_all_rows(qmv, n, k):
    run_case(qmv, synth.FMT_Q4_0, n, k, 1, synth.DT_F32, seed=0, expect_path=q4_path(1, k, n))


@pytest.mark.parametrize("m", [2, 4, 8])
@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_q4_0_full_size_batched_all_rows(qmv, n, k, m):
    # the batch workloads the benchmark times (K-chunked kernel), at their full sizes
    run_case(qmv, synth.FMT_Q4_0, n, k, m, synth.DT_F32, seed=m,
             expect_path=q4_path(m, k))


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


@pytest.mark.parametrize("n,k,m,xt", [(4, 2048 * 9, 1, synth.DT_F32), (33, 2048 * 9 + 96, 1, synth.DT_F32),
                                      (70, 11008, 2, synth.DT_F32), (70, 11008, 4, synth.DT_BF16),
                                      (41, 11008, 8, synth.DT_F32), (9, 4096, 8, synth.DT_BF16), (3, 64, 8, synth.DT_F32)])
def test_q4_0_k_chunked_batches(qmv, n, k, m, xt):
    # activations beyond one workgroup's LDS (m * k > 16384, or k > 16384) go through the
    # K-chunked kernel; the ragged last chunk and row tails are included
    run_case(qmv, synth.FMT_Q4_0, n, k, m, xt, seed=n + k + m, expect_path=q4_path(m, k))


def test_q4_0_chunked_unit_vector_returns_column_exactly(qmv):
    import torch
    n, k, m = 37, 11008, 3
    w = synth.gen_weights(synth.FMT_Q4_0, n, k, seed=15)
    W = qweights(synth.FMT_Q4_0, n, k, w)
    dense = oracle.dequant(oracle.Mat(synth.FMT_Q4_0, n, k, w)).astype(np.float32)
    cols = (0, 2047, 2048, 6000, 11007)
    e = np.zeros((m, k), dtype=np.float32)
    for r, j in enumerate(cols[:m]):
        e[r, j] = 1.0
    y = qmv.gemv(W, x_to_device(e, synth.DT_F32))
    torch.cuda.synchronize()
    assert qmv.last_path() == q4_path(m, k)
    y = y.cpu().numpy()
    for r, j in enumerate(cols[:m]):
        assert np.array_equal(y[r], dense[:, j]), j


# ------------------------------------------------------------------ q6_K

Q6_SMALL = [(1, 256), (3, 512), (37, 1024), (64, 2048), (100, 4096), (20, 11008), (10, 16384), (5, 768)]


@pytest.mark.parametrize("n,k", Q6_SMALL)
def test_q6k_small_full_parity(qmv, n, k):
    run_case(qmv, synth.FMT_Q6_K, n, k, 1, synth.DT_F32, seed=n + k)


def test_q6k_parity_config_256x1024_seed0(qmv):
    # the q6_K decode workload: 256 x 1024, four super-blocks per row, seed 0, all rows
    err = run_case(qmv, synth.FMT_Q6_K, 256, 1024, 1, synth.DT_F32, seed=0,
                   expect_path="q6_K.lds-x.fma-mix.rowgroup")
    print("max |err| / sum|w||x| =", err)


def q6_path(m, k):
    # one unit-dot per batch row up to batch 2 (fp16 codes converted inside the FMA), each
    # code converted once and applied to every row with fp32 FMAs from batch 3 up; rows of
    # fewer than 64 units that divide 64 go several to a wave; from batch 5 up 256-thread
    # workgroups over half chunks (two rows per wave)
    if m >= 5:
        return "q6_K.lds-x.fmac.wg256"
    base = "q6_K.lds-x.fmac" if m >= 3 else "q6_K.lds-x.fma-mix"
    return base + ".rowgroup" if k // 64 < 64 and 64 % (k // 64) == 0 else base


@pytest.mark.parametrize("m", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("xt", [synth.DT_F32, synth.DT_BF16])
def test_q6k_batched(qmv, m, xt):
    run_case(qmv, synth.FMT_Q6_K, 70, 2048, m, xt, seed=m + 100, expect_path=q6_path(m, 2048))


@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096)])
def test_q6k_large_all_rows(qmv, n, k):
    run_case(qmv, synth.FMT_Q6_K, n, k, 1, synth.DT_F32, seed=0)


@pytest.mark.parametrize("n,k,m,xt", [(4, 32768, 1, synth.DT_F32), (33, 20480, 1, synth.DT_F32),
                                      (70, 11008, 2, synth.DT_F32), (70, 11008, 4, synth.DT_BF16),
                                      (41, 11008, 8, synth.DT_F32), (9, 4352, 8, synth.DT_BF16),
                                      (17, 8192, 3, synth.DT_F32), (3, 256, 8, synth.DT_F32),
                                      (29, 4096, 4, synth.DT_F32), (13, 12288 + 256, 6, synth.DT_BF16),
                                      (8, 1024, 3, synth.DT_BF16), (64, 16384, 7, synth.DT_F32)])
def test_q6k_k_chunked_batches(qmv, n, k, m, xt):
    # K is walked 4096 activations at a time: one, two (even), three and five (odd) chunks,
    # ragged last chunks (11008 = 2 * 4096 + 2816, 4352 = 4096 + 256), batches up to 8
    run_case(qmv, synth.FMT_Q6_K, n, k, m, xt, seed=n + k + m, expect_path=q6_path(m, k))


@pytest.mark.parametrize("n,k,m,xt", [(41, 11008, 8, synth.DT_F32), (9, 4352, 5, synth.DT_BF16), (3, 256, 6, synth.DT_F32),
                                      (70, 3072, 7, synth.DT_F32), (13, 2048, 8, synth.DT_BF16)])
@pytest.mark.parametrize("path", ["default", "q6_K.wg512"])
def test_q6k_batch5_forms(qmv, monkeypatch, n, k, m, xt, path):
    # batches 5-8 in both workgroup forms: 32-unit chunks (ragged: 3072 = 48 units, 4352 =
    # 68), rows of one and four units per chunk, and the 512-thread form on request
    if path != "default":
        monkeypatch.setenv("QMV_FORCE_PATH", path)
        k64 = k // 64
        expect = "q6_K.lds-x.fmac.rowgroup" if k64 < 64 and 64 % k64 == 0 else "q6_K.lds-x.fmac"
    else:
        expect = q6_path(m, k)
    run_case(qmv, synth.FMT_Q6_K, n, k, m, xt, seed=n + k + m, expect_path=expect)


def test_q6k_chunked_unit_vector_returns_column_exactly(qmv):
    import torch
    n, k, m = 37, 11008, 5
    w = synth.gen_weights(synth.FMT_Q6_K, n, k, seed=16)
    W = qweights(synth.FMT_Q6_K, n, k, w)
    dense = oracle.dequant(oracle.Mat(synth.FMT_Q6_K, n, k, w)).astype(np.float32)
    cols = (0, 4095, 4096, 8200, 11007)  # chunk edges and the ragged last chunk
    e = np.zeros((m, k), dtype=np.float32)
    for r, j in enumerate(cols):
        e[r, j] = 1.0
    y = qmv.gemv(W, x_to_device(e, synth.DT_F32))
    torch.cuda.synchronize()
    assert qmv.last_path() == q6_path(m, k)
    y = y.cpu().numpy()
    for r, j in enumerate(cols):
        assert np.array_equal(y[r], dense[:, j]), j


def test_q6k_unit_vector_returns_column_exactly(qmv):
    import torch
    n, k = 96, 2048
    w = synth.gen_weights(synth.FMT_Q6_K, n, k, seed=7)
    W = qweights(synth.FMT_Q6_K, n, k, w)
    dense = oracle.dequant(oracle.Mat(synth.FMT_Q6_K, n, k, w))
    assert np.array_equal(dense.astype(np.float32).astype(np.float64), dense)  # exact in fp32
    for j in (0, 15, 16, 64, 100, 127, 128, 255, 256, 2047):
        e = np.zeros((1, k), dtype=np.float32)
        e[0, j] = 1.0
        y = qmv.gemv(W, x_to_device(e, synth.DT_F32))
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy()[0], dense[:, j].astype(np.float32)), j


def test_q6k_all_codes_32_give_zero(qmv):
    import torch
    n, k = 16, 1024
    w = synth.gen_weights(synth.FMT_Q6_K, n, k, seed=3)
    w["ql"][:] = 0x00
    w["qh"][:] = 0xAA  # every 2-bit field = 2, so q = 0 | 2 << 4 = 32
    W = qweights(synth.FMT_Q6_K, n, k, w)
    y = qmv.gemv(W, x_to_device(synth.gen_x(1, k, seed=3), synth.DT_F32))
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0.0)


def test_q4_0_all_codes_8_give_zero(qmv):
    # every weight is d * (8 - 8) = 0, so sum |w||x| = 0 and the output must be exactly 0
    import torch
    n, k = 40, 4096
    w = synth.gen_weights(synth.FMT_Q4_0, n, k, seed=2)
    w["qs"][:] = 0x88
    y = qmv.gemv(qweights(synth.FMT_Q4_0, n, k, w), x_to_device(synth.gen_x(1, k, seed=2), synth.DT_F32))
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0.0)


def test_q4_0_near_degenerate_rows_stay_within_bound(qmv):
    # rows that are zero except for a few weights: the error must stay relative to sum |w||x|
    n, k = 32, 8192
    w = synth.gen_weights(synth.FMT_Q4_0, n, k, seed=12)
    w["qs"][:] = 0x88
    rng = np.random.default_rng(12)
    for r in range(n):
        for b in rng.choice(k // 32, size=r % 4 + 1, replace=False):
            w["qs"][r, b, rng.integers(16)] = rng.integers(256)
    import torch
    x = synth.gen_x(1, k, seed=12) * np.float32(100.0)
    y = qmv.gemv(qweights(synth.FMT_Q4_0, n, k, w), x_to_device(x, synth.DT_F32))
    torch.cuda.synchronize()
    yr, b = oracle.gemv(oracle.Mat(synth.FMT_Q4_0, n, k, w), x)
    assert_parity(y.cpu().numpy(), yr, b, "near-degenerate q4_0")


# ------------------------------------------------------------- 4-bit codebook

CB4_SMALL = [(1, 128), (9, 384), (64, 2048), (77, 7168), (50, 11008 // 128 * 128), (13, 16384)]


@pytest.mark.parametrize("n,k", CB4_SMALL)
@pytest.mark.parametrize("xt", [synth.DT_BF16, synth.DT_F32])
def test_cb4_small_full_parity(qmv, n, k, xt):
    run_case(qmv, synth.FMT_CB4, n, k, 1, xt, seed=n + k, expect_path="cb4.lds-table.fma-mix")


@pytest.mark.parametrize("m", [2, 3, 4, 8])
def test_cb4_batched(qmv, m):
    # the one-shot kernel up to batch 2, the K-chunked one from batch 3 up
    path = "cb4.lds-f32-table-chunked.fmac" if m >= 3 else "cb4.lds-table.fma-mix"
    run_case(qmv, synth.FMT_CB4, 40, 2048, m, synth.DT_BF16, seed=m + 7, expect_path=path)


@pytest.mark.parametrize("n,k", [(2048, 7168), (7168, 2048)])
def test_cb4_expert_shapes_all_rows(qmv, n, k):
    run_case(qmv, synth.FMT_CB4, n, k, 1, synth.DT_BF16, seed=0)


@pytest.mark.parametrize("n,k,m,xt", [(4, 32768, 1, synth.DT_F32), (33, 20480, 1, synth.DT_BF16),
                                      (3, 16512, 1, synth.DT_F32), (70, 10880, 2, synth.DT_F32),
                                      (41, 7168, 8, synth.DT_BF16), (9, 4224, 5, synth.DT_F32),
                                      (2, 2176, 8, synth.DT_BF16), (17, 16384, 3, synth.DT_F32)])
def test_cb4_k_chunked_batches(qmv, n, k, m, xt):
    # K walked 2048 weights at a time: even and odd step counts, ragged last steps down to
    # one 128-weight group (16512 = 8 * 2048 + 128, 4224 = 2 * 2048 + 128), batches up to 8
    path = "cb4.lds-f32-table-chunked.fmac" if (m >= 3 or m * k > 16384 or k > 16384) else "cb4.lds-table.fma-mix"
    run_case(qmv, synth.FMT_CB4, n, k, m, xt, seed=n + k + m, expect_path=path)


@pytest.mark.parametrize("n,k,m,xt", [(1, 128, 1, synth.DT_F32), (9, 384, 3, synth.DT_BF16), (40, 2048, 4, synth.DT_F32),
                                      (65, 2176, 6, synth.DT_BF16), (23, 4096, 7, synth.DT_F32),
                                      (16, 2048, 8, synth.DT_BF16)])
def test_cb4_chunked_forced_small(qmv, monkeypatch, n, k, m, xt):
    # the K-chunked kernel where the one-shot kernel would run: one step, ragged single
    # steps, several batch rows
    monkeypatch.setenv("QMV_FORCE_PATH", "cb4.chunked")
    run_case(qmv, synth.FMT_CB4, n, k, m, xt, seed=n + k + m, expect_path="cb4.lds-f32-table-chunked.fmac")


def test_cb4_chunked_unit_vector_returns_codebook_entry_exactly(qmv):
    import torch
    n, k, m = 37, 10880, 5
    w = synth.gen_weights(synth.FMT_CB4, n, k, seed=17)
    W = qweights(synth.FMT_CB4, n, k, w)
    dense = oracle.dequant(oracle.Mat(synth.FMT_CB4, n, k, w)).astype(np.float32)
    cols = (0, 2047, 2048, 6001, 10879)  # step edges and the ragged last step
    e = np.zeros((m, k), dtype=np.float32)
    for r, j in enumerate(cols):
        e[r, j] = 1.0
    y = qmv.gemv(W, x_to_device(e, synth.DT_F32))
    torch.cuda.synchronize()
    assert qmv.last_path() == "cb4.lds-f32-table-chunked.fmac"
    y = y.cpu().numpy()
    for r, j in enumerate(cols):
        assert np.array_equal(y[r], dense[:, j]), j


def test_cb4_unit_vector_returns_codebook_entry_exactly(qmv):
    import torch
    n, k = 64, 1024
    w = synth.gen_weights(synth.FMT_CB4, n, k, seed=11)
    W = qweights(synth.FMT_CB4, n, k, w)
    dense = oracle.dequant(oracle.Mat(synth.FMT_CB4, n, k, w)).astype(np.float32)
    for j in (0, 1, 127, 128, 500, 1023):
        e = np.zeros((1, k), dtype=np.float32)
        e[0, j] = 1.0
        y = qmv.gemv(W, x_to_device(e, synth.DT_F32))
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy()[0], dense[:, j]), j


# ------------------------------------------------------------- 2-bit additive

AQ_SMALL = [(1, 8), (5, 24), (9, 64), (33, 1000), (64, 4096), (17, 4096 + 8), (40, 14336), (7, 12288),
            (5, 4160), (3, 8192 + 192)]


def aq_rows(m, n):
    # rows per wave of the streaming kernel: two for batches over at least 2 x 8 rows per CU
    # (4096 on 256 CUs), four at batch 8 over 4 x 8 rows per CU (8192); at batch 5-7 over
    # 2 x 16 rows per CU (8192) the half-step form, two rows per 32-lane group.  The
    # thresholds scale with the device's CU count, as the library's do.
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if 5 <= m <= 7 and n >= 32 * cus:
        return ".2row.half-step"
    return ".4row" if m >= 8 and n >= 32 * cus else ".2row" if m > 1 and n >= 16 * cus else ""


def aq_path(fmt, k, m=1, n=1):
    # the streaming kernel when k % 64 == 0, else the ragged one
    name = "aq2x8" if fmt == synth.FMT_AQ2X8 else "aq3x8"
    if k % 64:
        return f"{name}.ragged.lds-codebook.fma-mix"
    return f"{name}.stream.lds-codebook.fma-mix" + aq_rows(m, n)


@pytest.mark.parametrize("fmt", [synth.FMT_AQ2X8, synth.FMT_AQ3X8])
@pytest.mark.parametrize("n,k,m,xt", [(37, 4096 + 64, 5, synth.DT_BF16), (6, 2048, 8, synth.DT_F32),
                                      (19, 64, 6, synth.DT_BF16), (33, 8192 + 2048, 7, synth.DT_F32)])
@pytest.mark.parametrize("force", ["aq.half", "aq.wg512"])
def test_aq_batch5_forms(qmv, monkeypatch, fmt, n, k, m, xt, force):
    # batches 5-8 in the half-step form (two rows per 32-lane group, 2048-weight steps) and
    # in the full-step form on request: ragged steps, one unit, row counts not a multiple
    # of the 16 rows of a half-step workgroup
    monkeypatch.setenv("QMV_FORCE_PATH", force)
    name = "aq2x8" if fmt == synth.FMT_AQ2X8 else "aq3x8"
    expect = f"{name}.stream.lds-codebook.fma-mix" + (".2row.half-step" if force == "aq.half" else aq_rows(min(m, 4), n))
    run_case(qmv, fmt, n, k, m, xt, seed=n + k + m, expect_path=expect)


@pytest.mark.parametrize("n,k", AQ_SMALL)
def test_aq_small_full_parity(qmv, n, k):
    run_case(qmv, synth.FMT_AQ2X8, n, k, 1, synth.DT_BF16, seed=n + k, expect_path=aq_path(synth.FMT_AQ2X8, k))


@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 14336)])
def test_aq_config_shapes_all_rows(qmv, m, n, k):
    run_case(qmv, synth.FMT_AQ2X8, n, k, m, synth.DT_BF16, seed=0)


@pytest.mark.parametrize("m", [2, 3, 8])
def test_aq_batched_f32(qmv, m):
    run_case(qmv, synth.FMT_AQ2X8, 50, 2048, m, synth.DT_F32, seed=m + 3)


def test_aq_cancelling_codebooks_give_zero(qmv):
    # C2 = -C1: every weight is exactly 0 when c1 == c2, so the row must come out as 0
    import torch
    n, k = 24, 4096
    w = synth.gen_weights(synth.FMT_AQ2X8, n, k, seed=5)
    w["cbk"][1] = -w["cbk"][0]
    w["codes"][:, :, 1] = w["codes"][:, :, 0]
    y = qmv.gemv(qweights(synth.FMT_AQ2X8, n, k, w), x_to_device(synth.gen_x(1, k, synth.DT_BF16, seed=5), synth.DT_BF16))
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0.0)


def test_aq_single_codebook_vq_case(qmv):
    # C2 = 0 reduces the additive code to plain vector quantization
    n, k = 32, 2048
    w = synth.gen_weights(synth.FMT_AQ2X8, n, k, seed=6)
    w["cbk"][1] = 0
    import torch
    x = synth.gen_x(1, k, synth.DT_BF16, seed=6)
    y = qmv.gemv(qweights(synth.FMT_AQ2X8, n, k, w), x_to_device(x, synth.DT_BF16))
    torch.cuda.synchronize()
    yr, b = oracle.gemv(oracle.Mat(synth.FMT_AQ2X8, n, k, w), x, oracle.BF16)
    assert_parity(y.cpu().numpy(), yr, b, "aq vq")


@pytest.mark.parametrize("m,xt", [(5, synth.DT_BF16), (8, synth.DT_F32)])
def test_aq_batched_multi_step(qmv, m, xt):
    # more than four batch rows: one activation buffer, two barriers per step; 3 steps
    run_case(qmv, synth.FMT_AQ2X8, 19, 12288, m, xt, seed=m + 31, expect_path=aq_path(synth.FMT_AQ2X8, 12288, m))


# ------------------------------------------------------------- 3-bit additive

@pytest.mark.parametrize("fmt", [synth.FMT_AQ2X8, synth.FMT_AQ3X8])
@pytest.mark.parametrize("force,m,n", [("aq.r2", 1, 37), ("aq.r1", 4, 37), ("", 3, 17), ("", 3, 4096 + 17),
                                       ("aq.r2", 2, 1), ("aq.r4", 1, 37), ("aq.r4", 4, 203), ("aq.r4", 8, 6),
                                       ("", 8, 8192 + 17), ("", 6, 8192 + 17)])
def test_aq_rows_per_wave(qmv, monkeypatch, fmt, force, m, n):
    # one, two or four rows per wave, forced or by default; row counts that are not a multiple
    # of the rows per workgroup leave the last wave's later rows past the end
    if force:
        monkeypatch.setenv("QMV_FORCE_PATH", force)
    k = 4096 + 64
    name = "aq2x8" if fmt == synth.FMT_AQ2X8 else "aq3x8"
    rows = {"aq.r1": "", "aq.r2": ".2row", "aq.r4": ".4row"}.get(force, aq_rows(m, n))
    run_case(qmv, fmt, n, k, m, synth.DT_F32, seed=n + m,
             expect_path=f"{name}.stream.lds-codebook.fma-mix" + rows)


@pytest.mark.parametrize("n,k", AQ_SMALL)
def test_aq3_small_full_parity(qmv, n, k):
    run_case(qmv, synth.FMT_AQ3X8, n, k, 1, synth.DT_BF16, seed=n + k + 1, expect_path=aq_path(synth.FMT_AQ3X8, k))


@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 14336)])
def test_aq3_config_shapes_all_rows(qmv, m, n, k):
    run_case(qmv, synth.FMT_AQ3X8, n, k, m, synth.DT_BF16, seed=0)


@pytest.mark.parametrize("m,xt,k", [(2, synth.DT_F32, 2048), (3, synth.DT_BF16, 8192 + 64), (6, synth.DT_F32, 12288),
                                    (8, synth.DT_BF16, 4096), (4, synth.DT_F32, 1000)])
def test_aq3_batched(qmv, m, xt, k):
    run_case(qmv, synth.FMT_AQ3X8, 37, k, m, xt, seed=m + 13, expect_path=aq_path(synth.FMT_AQ3X8, k, m))


def test_aq3_cancelling_codebooks_give_zero(qmv):
    # C2 = -C1 and C3 = 0: every weight is exactly 0 when c1 == c2
    import torch
    n, k = 24, 8192
    w = synth.gen_weights(synth.FMT_AQ3X8, n, k, seed=5)
    w["cbk"][1] = -w["cbk"][0]
    w["cbk"][2] = 0
    w["codes"][:, :, 1] = w["codes"][:, :, 0]
    y = qmv.gemv(qweights(synth.FMT_AQ3X8, n, k, w), x_to_device(synth.gen_x(2, k, synth.DT_BF16, seed=5), synth.DT_BF16))
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0.0)


def test_aq3_with_zero_third_codebook_matches_two_codebook_kernel(qmv):
    # C3 = 0: the 3-book kernel on (c1, c2, c3) and the 2-book kernel on (c1, c2) compute
    # the same weights; both are held to the oracle and to each other within the bound
    import torch
    n, k = 40, 4096 * 2
    w3 = synth.gen_weights(synth.FMT_AQ3X8, n, k, seed=9)
    w3["cbk"][2] = 0
    w2 = {"codes": np.ascontiguousarray(w3["codes"][:, :, :2]), "cbk": np.ascontiguousarray(w3["cbk"][:2]),
          "s": w3["s"]}
    x = synth.gen_x(1, k, synth.DT_F32, seed=9)
    y3 = qmv.gemv(qweights(synth.FMT_AQ3X8, n, k, w3), x_to_device(x, synth.DT_F32))
    y2 = qmv.gemv(qweights(synth.FMT_AQ2X8, n, k, w2), x_to_device(x, synth.DT_F32))
    torch.cuda.synchronize()
    yr, b = oracle.gemv(oracle.Mat(synth.FMT_AQ3X8, n, k, w3), x, oracle.F32)
    assert_parity(y3.cpu().numpy(), yr, b, "aq3 c3=0")
    assert_parity(y2.cpu().numpy(), yr, b, "aq2 same weights")


# ------------------------------------------------------------- 8-bit codebook

CB8_SMALL = [(1, 64), (9, 192), (33, 4096), (17, 4160), (5, 12288), (40, 7168), (3, 16384 + 64)]


@pytest.mark.parametrize("n,k", CB8_SMALL)
@pytest.mark.parametrize("xt", [synth.DT_BF16, synth.DT_F32])
def test_cb8_small_full_parity(qmv, n, k, xt):
    run_case(qmv, synth.FMT_CB8, n, k, 1, xt, seed=n + k, expect_path="cb8.stream.lds-table.fma-mix")


@pytest.mark.parametrize("m,xt,k", [(2, synth.DT_BF16, 2048), (3, synth.DT_F32, 7168), (4, synth.DT_BF16, 12288),
                                    (5, synth.DT_F32, 4160), (8, synth.DT_BF16, 7168), (6, synth.DT_F32, 16384 + 64),
                                    (7, synth.DT_BF16, 64), (4, synth.DT_F32, 4096), (3, synth.DT_BF16, 4160)])
def test_cb8_batched(qmv, m, xt, k):
    run_case(qmv, synth.FMT_CB8, 29, k, m, xt, seed=m + 17, expect_path=cb8_path(m, 29))


def cb8_path(m, n=0, force=None):
    # fp16 codebook slice at batch 1, 2 and 4; fp32 slice at 3 and from 5 up, where the
    # half-step form (two rows per wave, 2048-weight steps) runs on matrices of at least 16
    # rows per CU, or when forced
    import torch
    if m >= 5:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        half = force == "cb8.half" or (force is None and n >= 16 * cus)
        return "cb8.stream.lds-f32-table.fmac.half-step" if half else "cb8.stream.lds-f32-table.fmac"
    return "cb8.stream.lds-f32-table.fmac" if m == 3 else "cb8.stream.lds-table.fma-mix"


@pytest.mark.parametrize("n,k,m,xt", [(29, 7168, 8, synth.DT_BF16), (17, 2048 + 64, 5, synth.DT_F32),
                                      (3, 64, 6, synth.DT_BF16), (40, 16384 + 64, 7, synth.DT_F32),
                                      (2048, 7168, 8, synth.DT_BF16), (7168, 2048, 6, synth.DT_BF16)])
@pytest.mark.parametrize("path", ["default", "cb8.half", "cb8.wg512"])
def test_cb8_batch5_forms(qmv, monkeypatch, n, k, m, xt, path):
    # batches 5-8 in both forms: ragged half steps (2112 = 2048 + 64), a single unit, odd
    # row counts (a wave's second row past n), full-size shapes on sampled rows
    force = None if path == "default" else path
    if force:
        monkeypatch.setenv("QMV_FORCE_PATH", force)
    run_case(qmv, synth.FMT_CB8, n, k, m, xt, seed=n + k + m, expect_path=cb8_path(m, n, force))


@pytest.mark.parametrize("n,k", [(2048, 7168), (7168, 2048), (129280, 7168)])
def test_cb8_shared_expert_and_head_shapes_all_rows(qmv, n, k):
    # the shared expert's gate/up and down, and the output head, at their full sizes
    run_case(qmv, synth.FMT_CB8, n, k, 1, synth.DT_BF16, seed=0)


def test_cb8_unit_vector_returns_codebook_entry_exactly(qmv):
    import torch
    n, k, m = 45, 8192 + 128, 6
    w = synth.gen_weights(synth.FMT_CB8, n, k, seed=21)
    dense = oracle.dequant(oracle.Mat(synth.FMT_CB8, n, k, w)).astype(np.float32)
    cols = (0, 63, 4095, 4096, 8191, 8319)  # unit and step edges, the ragged last step
    e = np.zeros((m, k), dtype=np.float32)
    for r, j in enumerate(cols):
        e[r, j] = 1.0
    y = qmv.gemv(qweights(synth.FMT_CB8, n, k, w), x_to_device(e, synth.DT_F32))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    for r, j in enumerate(cols):
        assert np.array_equal(y[r], dense[:, j]), j


def test_binding_rejects_bad_tensors(qmv):
    # wrong layout, shape or dtype never reaches the library as a bare address
    import torch
    n, k = 8, 64
    w = synth.gen_weights(synth.FMT_Q4_0, n, k, seed=3)
    W = qweights(synth.FMT_Q4_0, n, k, w)
    x = torch.zeros(k, 2, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="contiguous"):
        qmv.gemv(W, x.t())
    with pytest.raises(ValueError, match="shape"):
        qmv.gemv(W, torch.zeros(1, k + 32, device="cuda"))
    with pytest.raises(ValueError, match="shape"):
        qmv.gemv(W, torch.zeros(2, k, device="cuda"), y=torch.empty(2, n - 1, device="cuda"))
    with pytest.raises(TypeError):
        qmv.gemv(W, torch.zeros(1, k, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError, match="bytes"):
        qmv.QWeights(synth.FMT_Q4_0, n, k, {"qs": W.planes["qs"][:-1], "d": W.planes["d"]})
    y = qmv.gemv(W, torch.zeros(2, k, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (2, n) and not y.abs().sum().item()
