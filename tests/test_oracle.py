"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-worked fixture under
tests/golden/ (with its citation), a library routine (numpy), exact rational
arithmetic, or a closed form.  None of these tests needs a GPU.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            toks = val.split()
            conv = [int(t, 16) if t.startswith("0x") else (int(t) if t.lstrip("-").isdigit() else float(t))
                    for t in toks]
            out[key] = conv if len(conv) > 1 else conv[0]
    return out


def f16(v):
    return np.array(v, dtype=np.float64).astype(np.float16)


# ----------------------------------------------------------------- scalars

def test_f16_decode_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_bf16_decode_matches_float32_upper_half():
    bits = np.arange(0, 65536, 7, dtype=np.uint32)
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)  # noqa
    got = np.array([oracle.bf16(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
    assert abs(oracle.silu(-1.0) + 1.0 / (1.0 + np.e)) < 1e-15
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15


# ------------------------------------------------------------ layout fixtures

def test_q4_0_golden_block():
    g = load_golden("q4_0_block.txt")
    qs = np.array(g["bytes"], dtype=np.uint8).reshape(1, 1, 16)
    d = np.array([g["d_bits"]], dtype=np.uint16).view(np.float16).reshape(1, 1)
    m = oracle.Mat(oracle.Q4_0, 1, 32, {"qs": qs, "d": d})
    assert oracle.codes(m)[0].tolist() == g["codes"]
    assert oracle.dequant(m)[0].tolist() == [float(w) for w in g["weights"]]
    blk = oracle.q4_0_to_blocks(qs, d)
    assert blk.tolist() == g["block18"]
    qs2, d2 = oracle.q4_0_from_blocks(blk)
    assert np.array_equal(qs2, qs.ravel()) and np.array_equal(d2.view(np.uint16), d.ravel().view(np.uint16))


def _golden_q6k():
    g = load_golden("q6k_superblock.txt")
    ql = np.arange(128, dtype=np.uint8).reshape(1, 1, 128)
    qh = np.full((1, 1, 64), g["qh_byte"], dtype=np.uint8)
    sc = (np.arange(16) + 1).astype(np.int8).reshape(1, 1, 16)
    d = np.array([g["d_bits"]], dtype=np.uint16).view(np.float16).reshape(1, 1)
    return g, oracle.Mat(oracle.Q6_K, 1, 256, {"ql": ql, "qh": qh, "sc": sc, "d": d})


def test_q6k_golden_superblock():
    g, m = _golden_q6k()
    c = oracle.codes(m)[0]
    w = oracle.dequant(m)[0]
    pos = g["positions"]
    assert [int(c[p]) for p in pos] == g["codes"]
    assert [float(w[p]) for p in pos] == [float(v) for v in g["weights"]]
    blk = oracle.q6k_to_blocks(m.planes["ql"], m.planes["qh"], m.planes["sc"], m.planes["d"])
    assert blk.size == 210
    o_ql, o_qh, o_sc, o_d = g["block_offsets"]
    assert blk[o_ql:o_ql + 128].tolist() == list(range(128))
    assert set(blk[o_qh:o_qh + 64].tolist()) == {g["qh_byte"]}
    assert blk[o_sc:o_sc + 16].tolist() == list(range(1, 17))
    assert blk[o_d:o_d + 2].tolist() == [0x00, 0x3C]
    ql, qh, sc, d = oracle.q6k_from_blocks(blk)
    assert np.array_equal(ql, m.planes["ql"].ravel()) and np.array_equal(qh, m.planes["qh"].ravel())
    assert np.array_equal(sc, m.planes["sc"].ravel())


def test_cb4_golden_group():
    g = load_golden("cb4_group.txt")
    i = np.arange(64)
    idx = ((i % 16) | ((15 - i % 16) << 4)).astype(np.uint8).reshape(1, 64)
    cb = f16(np.arange(16) / 16.0).reshape(1, 1, 16)
    m = oracle.Mat(oracle.CB4, 1, 128, {"idx": idx, "cb": cb})
    w = oracle.dequant(m)[0]
    assert [float(w[p]) for p in g["positions"]] == [float(v) for v in g["weights"]]


def test_aq_golden_group():
    g = load_golden("aq_group.txt")
    codes = np.array([[[g["c1"], g["c2"]]]], dtype=np.uint8)
    cbk = np.zeros((2, 256, 8), dtype=np.float16)
    cbk[0, g["c1"]] = f16((np.arange(8) + 1) / 8.0)
    cbk[1, g["c2"]] = f16(-np.arange(8) / 4.0)
    s = np.array([g["s_bits"]], dtype=np.uint16).view(np.float16)
    m = oracle.Mat(oracle.AQ2X8, 1, 8, {"codes": codes, "cbk": cbk, "s": s})
    assert oracle.dequant(m)[0].tolist() == [float(v) for v in g["weights"]]


def test_cb8_golden_row():
    g = load_golden("cb8_row.txt")
    idx = np.array(g["idx"], dtype=np.uint8).reshape(1, 16)
    cb = f16((np.arange(256) - 128) / 64.0).reshape(1, 256)
    m = oracle.Mat(oracle.CB8, 1, 16, {"idx": idx, "cb": cb})
    assert oracle.dequant(m)[0].tolist() == [float(v) for v in g["weights"]]
    assert oracle.codes(m)[0].tolist() == g["idx"]


def test_aq3_golden_group():
    g = load_golden("aq3_group.txt")
    codes = np.array([[[g["c1"], g["c2"], g["c3"]]]], dtype=np.uint8)
    cbk = np.zeros((3, 256, 8), dtype=np.float16)
    cbk[0, g["c1"]] = f16(np.arange(8) / 2.0)
    cbk[1, g["c2"]] = f16(-0.25 * np.ones(8))
    cbk[2, g["c3"]] = f16((8 - np.arange(8)) / 16.0)
    s = np.array([g["s_bits"]], dtype=np.uint16).view(np.float16)
    m = oracle.Mat(oracle.AQ3X8, 1, 8, {"codes": codes, "cbk": cbk, "s": s})
    assert oracle.dequant(m)[0].tolist() == [float(v) for v in g["weights"]]


# -------------------------------------------------------------- round trips

def test_q4_0_round_trip_exhaustive():
    # every nibble value at every position of a block
    q = np.array([[(v + p) % 16 for p in range(32)] for v in range(16)], dtype=np.int32)
    q = q.reshape(16, 32)
    qs = oracle.pack_q4_0(q)
    d = f16(np.ones((16, 1)))
    m = oracle.Mat(oracle.Q4_0, 16, 32, {"qs": qs, "d": d})
    assert np.array_equal(oracle.codes(m), q)
    # bytes -> codes -> bytes
    w = synth.gen_weights(synth.FMT_Q4_0, 8, 256, seed=3)
    m = oracle.Mat(oracle.Q4_0, 8, 256, w)
    assert np.array_equal(oracle.pack_q4_0(oracle.codes(m)), w["qs"])


def test_q6k_round_trip_exhaustive():
    # every 6-bit value at every position of four super-blocks
    q = np.array([[(v + p) % 64 for p in range(1024)] for v in range(64)], dtype=np.int32)
    ql, qh = oracle.pack_q6k(q)
    sc = np.ones((64, 4, 16), dtype=np.int8)
    d = f16(np.ones((64, 4)))
    m = oracle.Mat(oracle.Q6_K, 64, 1024, {"ql": ql, "qh": qh, "sc": sc, "d": d})
    assert np.array_equal(oracle.codes(m), q)
    w = synth.gen_weights(synth.FMT_Q6_K, 4, 1024, seed=5)
    m = oracle.Mat(oracle.Q6_K, 4, 1024, w)
    ql2, qh2 = oracle.pack_q6k(oracle.codes(m))
    assert np.array_equal(ql2, w["ql"]) and np.array_equal(qh2, w["qh"])


def test_cb4_round_trip():
    q = np.array([[(v * 7 + p) % 16 for p in range(256)] for v in range(16)], dtype=np.int32)
    idx = oracle.pack_cb4(q)
    cb = f16(np.zeros((16, 2, 16)))
    m = oracle.Mat(oracle.CB4, 16, 256, {"idx": idx, "cb": cb})
    assert np.array_equal(oracle.codes(m), q)


def test_aq_every_code_pair_reaches_its_rows():
    # C1[c][j] = c + j/8 and C2[c][j] = -c*2^-10: every (c1, c2) pair decodes to a unique vector
    n = 256
    cbk = np.zeros((2, 256, 8), dtype=np.float64)
    cbk[0] = np.arange(256)[:, None] + np.arange(8)[None, :] / 8.0
    cbk[1] = -np.arange(256)[:, None] * 2.0 ** -10
    cbk = f16(cbk)
    codes = np.stack([np.arange(n), (np.arange(n) * 37 + 11) % 256], axis=1).astype(np.uint8).reshape(n, 1, 2)
    s = f16(np.ones(n))
    m = oracle.Mat(oracle.AQ2X8, n, 8, {"codes": codes, "cbk": cbk, "s": s})
    w = oracle.dequant(m)
    ref = cbk[0, codes[:, 0, 0]].astype(np.float64) + cbk[1, codes[:, 0, 1]].astype(np.float64)
    assert np.array_equal(w, ref)


def test_cb8_every_index_at_every_position():
    # row v has index (v + p) % 256 at position p: every byte value at every position
    n, k = 256, 512
    q = np.array([[(v + p) % 256 for p in range(k)] for v in range(n)], dtype=np.int32)
    cb = f16(np.arange(n)[:, None] * 0 + (np.arange(256)[None, :] - 100) / 32.0)
    m = oracle.Mat(oracle.CB8, n, k, {"idx": q.astype(np.uint8), "cb": cb})
    assert np.array_equal(oracle.codes(m), q)
    assert np.array_equal(oracle.dequant(m), (q - 100) / 32.0)


def test_aq3_every_code_triple_reaches_its_rows():
    # C1[c][j] = c + j/8, C2[c][j] = -c*2^-10, C3[c][j] = c*2^-4 - j: each row's triple decodes
    # to the numpy sum of the three fp16 table rows times s
    n = 256
    cbk = np.zeros((3, 256, 8), dtype=np.float64)
    cbk[0] = np.arange(256)[:, None] + np.arange(8)[None, :] / 8.0
    cbk[1] = -np.arange(256)[:, None] * 2.0 ** -10
    cbk[2] = np.arange(256)[:, None] * 2.0 ** -4 - np.arange(8)[None, :]
    cbk = f16(cbk)
    r = np.arange(n)
    codes = np.stack([r, (r * 37 + 11) % 256, (r * 101 + 3) % 256], axis=1).astype(np.uint8).reshape(n, 1, 3)
    s = f16(0.5 + (r % 7) / 8.0)
    m = oracle.Mat(oracle.AQ3X8, n, 8, {"codes": codes, "cbk": cbk, "s": s})
    ref = (cbk[0, codes[:, 0, 0]].astype(np.float64) + cbk[1, codes[:, 0, 1]].astype(np.float64)
           + cbk[2, codes[:, 0, 2]].astype(np.float64)) * s.astype(np.float64)[:, None]
    assert np.array_equal(oracle.dequant(m), ref)


def test_aq3_with_zero_third_codebook_is_the_two_codebook_format():
    # C3 = 0 reduces the 3-bit code to the (separately pinned) 2-bit code over (c1, c2)
    w3 = synth.gen_weights(synth.FMT_AQ3X8, 5, 96, seed=12)
    w3["cbk"][2] = 0
    w2 = {"codes": np.ascontiguousarray(w3["codes"][:, :, :2]), "cbk": np.ascontiguousarray(w3["cbk"][:2]),
          "s": w3["s"]}
    m3, m2 = oracle.Mat(oracle.AQ3X8, 5, 96, w3), oracle.Mat(oracle.AQ2X8, 5, 96, w2)
    assert np.array_equal(oracle.dequant(m3), oracle.dequant(m2))
    x = synth.gen_x(2, 96, synth.DT_BF16, seed=12)
    assert np.array_equal(oracle.gemv(m3, x, oracle.BF16)[0], oracle.gemv(m2, x, oracle.BF16)[0])


# --------------------------------------------------------- GEMV arithmetic

def _dense_from_codes(fmt, q, planes):
    """The weight matrix built from codes the test chose (not from stored bytes)."""
    if fmt == oracle.Q4_0:
        d = planes["d"].astype(np.float64)
        return np.repeat(d, 32, axis=1) * (q - 8)
    if fmt == oracle.Q6_K:
        n, k = q.shape
        d = np.repeat(planes["d"].astype(np.float64), 256, axis=1)
        sc = np.repeat(planes["sc"].reshape(n, k // 16).astype(np.float64), 16, axis=1)
        return d * sc * (q - 32)
    if fmt == oracle.CB4:
        n, k = q.shape
        cb = planes["cb"].astype(np.float64)
        g = np.arange(k) // 128
        return cb[np.arange(n)[:, None], g[None, :], q]
    if fmt == oracle.CB8:
        n, k = q.shape
        return planes["cb"].astype(np.float64)[np.arange(n)[:, None], q]
    raise ValueError


@pytest.mark.parametrize("fmt,n,k", [(oracle.Q4_0, 13, 96), (oracle.Q6_K, 7, 512), (oracle.CB4, 9, 384),
                                     (oracle.CB8, 11, 160)])
@pytest.mark.parametrize("xt", [oracle.F32, oracle.BF16])
def test_gemv_matches_numpy_matmul(fmt, n, k, xt):
    rng = np.random.default_rng(11)
    if fmt == oracle.Q4_0:
        q = rng.integers(0, 16, (n, k)).astype(np.int32)
        planes = {"qs": oracle.pack_q4_0(q), "d": f16(rng.uniform(0.01, 0.02, (n, k // 32)))}
    elif fmt == oracle.Q6_K:
        q = rng.integers(0, 64, (n, k)).astype(np.int32)
        ql, qh = oracle.pack_q6k(q)
        planes = {"ql": ql, "qh": qh, "sc": rng.integers(-128, 128, (n, k // 256, 16)).astype(np.int8),
                  "d": f16(rng.uniform(1e-5, 1e-4, (n, k // 256)))}
    elif fmt == oracle.CB4:
        q = rng.integers(0, 16, (n, k)).astype(np.int32)
        planes = {"idx": oracle.pack_cb4(q), "cb": f16(np.sort(rng.normal(0, 0.02, (n, k // 128, 16)), axis=2))}
    else:
        q = rng.integers(0, 256, (n, k)).astype(np.int32)
        planes = {"idx": q.astype(np.uint8), "cb": f16(np.sort(rng.normal(0, 0.02, (n, 256)), axis=1))}
    m = oracle.Mat(fmt, n, k, planes)
    W = _dense_from_codes(fmt, q, planes)
    assert np.array_equal(oracle.dequant(m), W)
    xf = rng.standard_normal((3, k)).astype(np.float32)
    if xt == oracle.F32:
        x, xd = xf, xf.astype(np.float64)
    else:
        x = synth.f32_to_bf16_bits(xf)
        xd = synth.bf16_bits_to_f32(x).astype(np.float64)
    y, b = oracle.gemv(m, x, xt)
    ref = xd @ W.T
    assert y.shape == (3, n)
    assert np.all(np.abs(y - ref) <= 1e-13 * (np.abs(xd) @ np.abs(W).T))
    assert np.allclose(b, np.abs(xd) @ np.abs(W).T, rtol=1e-13, atol=0)


def test_gemv_exact_rational_tiny():
    w = synth.gen_weights(synth.FMT_AQ2X8, 3, 16, seed=2)
    m = oracle.Mat(oracle.AQ2X8, 3, 16, w)
    x = synth.gen_x(1, 16, synth.DT_BF16, seed=2)
    y, b = oracle.gemv(m, x, oracle.BF16)
    xd = synth.bf16_bits_to_f32(x[0]).astype(np.float64)
    for r in range(3):
        s = Fraction(float(w["s"][r]))
        exact = Fraction(0)
        for c in range(16):
            g, j = divmod(c, 8)
            c1, c2 = w["codes"][r, g]
            wv = s * (Fraction(float(w["cbk"][0, c1, j])) + Fraction(float(w["cbk"][1, c2, j])))
            exact += wv * Fraction(float(xd[c]))
        assert abs(Fraction(y[0, r]) - exact) <= Fraction(1e-14) * Fraction(b[0, r])


def test_aq3_gemv_exact_rational_tiny():
    w = synth.gen_weights(synth.FMT_AQ3X8, 3, 24, seed=4)
    m = oracle.Mat(oracle.AQ3X8, 3, 24, w)
    x = synth.gen_x(2, 24, synth.DT_F32, seed=4)
    y, b = oracle.gemv(m, x, oracle.F32)
    for bi in range(2):
        for r in range(3):
            s = Fraction(float(w["s"][r]))
            exact = Fraction(0)
            for c in range(24):
                g, j = divmod(c, 8)
                wv = s * sum(Fraction(float(w["cbk"][t, w["codes"][r, g, t], j])) for t in range(3))
                exact += wv * Fraction(float(x[bi, c]))
            assert abs(Fraction(y[bi, r]) - exact) <= Fraction(1e-14) * Fraction(b[bi, r])


def test_cb8_closed_forms():
    # one index per row: y = cb[row][v] * sum(x)   ("row-sum times scale"); x = e_j gives column j
    n, k = 6, 48
    v = np.array([0, 17, 128, 200, 255, 99])
    cb = f16(np.sort(np.random.default_rng(3).normal(0, 0.02, (n, 256)), axis=1))
    m = oracle.Mat(oracle.CB8, n, k, {"idx": np.repeat(v[:, None], k, axis=1).astype(np.uint8), "cb": cb})
    x = synth.gen_x(1, k, seed=6)
    y, _ = oracle.gemv(m, x)
    sx = float(np.sum(x[0].astype(np.float64)))
    for r in range(n):
        assert abs(y[0, r] - float(cb[r, v[r]]) * sx) <= 1e-15 * float(np.sum(np.abs(x)))
    w = synth.gen_weights(synth.FMT_CB8, 5, 48, seed=2)
    m = oracle.Mat(oracle.CB8, 5, 48, w)
    for j in (0, 13, 47):
        e = np.zeros((1, 48), dtype=np.float32)
        e[0, j] = 1.0
        assert np.array_equal(oracle.gemv(m, e)[0][0], w["cb"].astype(np.float64)[np.arange(5), w["idx"][:, j]])


def test_gemv_closed_forms():
    n, k = 5, 128
    # constant codes with one scale per row: y = scale * (c - 8) * sum(x)   ("row-sum times scale")
    q = np.full((n, k), 11, dtype=np.int32)
    d = f16(np.arange(1, n + 1)[:, None] * np.ones((n, k // 32)) / 64)
    m = oracle.Mat(oracle.Q4_0, n, k, {"qs": oracle.pack_q4_0(q), "d": d})
    x = synth.gen_x(1, k, seed=4)
    y, _ = oracle.gemv(m, x)
    sx = float(np.sum(x[0].astype(np.float64)))
    for r in range(n):
        assert abs(y[0, r] - (r + 1) / 64 * 3 * sx) <= 1e-13 * np.sum(np.abs(x))
    # x = e_j returns column j exactly
    w = synth.gen_weights(synth.FMT_Q6_K, 4, 512, seed=1)
    m = oracle.Mat(oracle.Q6_K, 4, 512, w)
    W = oracle.dequant(m)
    for j in (0, 77, 255, 256, 511):
        e = np.zeros((1, 512), dtype=np.float32)
        e[0, j] = 1.0
        y, _ = oracle.gemv(m, e)
        assert np.array_equal(y[0], W[:, j])
    # q6_K with every code 32 is zero; scaling x by 2 scales y by exactly 2
    q = np.full((4, 512), 32, dtype=np.int32)
    ql, qh = oracle.pack_q6k(q)
    mz = oracle.Mat(oracle.Q6_K, 4, 512, {"ql": ql, "qh": qh, "sc": w["sc"], "d": w["d"]})
    x = synth.gen_x(2, 512, seed=9)
    y, _ = oracle.gemv(mz, x)
    assert np.all(y == 0.0)
    y1, _ = oracle.gemv(m, x)
    y2, _ = oracle.gemv(m, (2 * x).astype(np.float32))
    assert np.array_equal(y2, 2 * y1)


def test_gemv_row_permutation_and_row_sampling():
    w = synth.gen_weights(synth.FMT_CB4, 6, 256, seed=8)
    m = oracle.Mat(oracle.CB4, 6, 256, w)
    perm = np.array([3, 0, 5, 1, 4, 2])
    mp = oracle.Mat(oracle.CB4, 6, 256, {"idx": w["idx"][perm], "cb": w["cb"][perm]})
    x = synth.gen_x(1, 256, synth.DT_BF16, seed=8)
    y, _ = oracle.gemv(m, x, oracle.BF16)
    yp, _ = oracle.gemv(mp, x, oracle.BF16)
    assert np.array_equal(yp[0], y[0, perm])
    ys, _ = oracle.gemv(m, x, oracle.BF16, rows=[5, 2])
    assert np.array_equal(ys[0], y[0, [5, 2]])


def test_aq_single_codebook_special_case():
    # C2 = 0 turns the additive code into plain vector quantization: w = s * C1[c1]
    w = synth.gen_weights(synth.FMT_AQ2X8, 4, 64, seed=6)
    w["cbk"][1] = 0
    m = oracle.Mat(oracle.AQ2X8, 4, 64, w)
    W = oracle.dequant(m)
    c1 = w["codes"][:, :, 0]
    ref = w["s"].astype(np.float64)[:, None] * w["cbk"][0][c1].astype(np.float64).reshape(4, 64)
    assert np.array_equal(W, ref)


# ------------------------------------------------------- activation quantizer

def test_quantizer_golden_blocks():
    g = load_golden("quant_act.txt")
    x = np.concatenate([np.array(g["a_x"], dtype=np.float32), np.zeros(32, np.float32),
                        np.array(g["c_x"], dtype=np.float32)])[None, :]
    assert np.float32(0.49999997).view(np.uint32) == 0x3EFFFFFF
    xq, xs = oracle.quant_act(x)
    assert xs[0].tolist() == [g["a_xs"], g["b_xs"], g["c_xs"]]
    assert xq[0, :32].tolist() == g["a_xq"]
    assert xq[0, 32:64].tolist() == [0] * 32
    assert xq[0, 64:].tolist() == g["c_xq"]


def test_quantizer_properties_random():
    x = synth.gen_x(4, 512, seed=12)
    xq, xs = oracle.quant_act(x)
    blocks = x.reshape(4, 16, 32)
    amax = np.max(np.abs(blocks), axis=2)
    assert np.array_equal(xs, (amax / np.float32(127)).astype(np.float32))
    q = xq.reshape(4, 16, 32).astype(np.int64)
    assert np.all(np.abs(q) <= 127)
    # the element holding the block maximum maps to +-127
    am = np.argmax(np.abs(blocks), axis=2)
    top = np.take_along_axis(q, am[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top) == 127)
    # |x/xs - xq| <= 1/2, and sign agrees
    r = blocks.astype(np.float64) / xs[..., None].astype(np.float64)
    assert np.all(np.abs(r - q) <= 0.5 + 1e-5)
    # negating x negates xq exactly (round half away from zero is odd-symmetric)
    xqn, xsn = oracle.quant_act(-x)
    assert np.array_equal(xqn, -xq) and np.array_equal(xsn, xs)


def _binary32_half_ulp(v: Fraction) -> Fraction:
    """Half the spacing of binary32 values around the positive value v (normal range)."""
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    return Fraction(2) ** (e - 24)


def test_quantizer_division_trap_block():
    # A block whose quotients round, in binary32, to exactly k + 1/2, so xq must be k + 1
    # (away from zero).  On the marked elements an oracle that divided in binary64 (the
    # exact quotient is below k + 1/2) or multiplied by fl32(1/xs) (the product lands
    # below k + 1/2) would give k.
    g = load_golden("quant_act.txt")
    x = np.array(g["d_x_bits"], dtype=np.uint32).view(np.float32)
    xs = np.uint32(g["d_xs_bits"]).view(np.float32)
    # xs itself: amax / 127 rounded to binary32 (exact rational check of the golden's claim)
    amax = Fraction(float(x[0]))
    assert abs(Fraction(float(xs)) - amax / 127) <= _binary32_half_ulp(amax / 127)
    recip = np.float32(1) / xs  # numpy binary32 division (correctly rounded)
    for i, (k, trap) in enumerate(zip(g["d_k"], g["d_trap"]), start=1):
        half = Fraction(2 * abs(k) + 1, 2)
        q = Fraction(float(abs(x[i]))) / Fraction(float(xs))
        assert abs(half - q) < _binary32_half_ulp(half)   # rounds to k + 1/2 in binary32
        if trap & 1:                                      # ... from below: the exact (or
            assert q < half                               # binary64) quotient rounds to k
        if trap & 2:                                      # the reciprocal form lands below
            assert Fraction(float(np.float32(abs(x[i])) * recip)) < half
    xq, xs_o = oracle.quant_act(x[None, :])
    assert xs_o.view(np.uint32)[0, 0] == g["d_xs_bits"]
    assert xq[0].tolist() == g["d_xq"]


def test_quantizer_matches_numpy_binary32_reference():
    # numpy's own binary32 arithmetic over a full activation matrix of the prefill workload:
    # amax and the two divisions in float32 (IEEE, correctly rounded), the rounding to an
    # integer done exactly in float64 (trunc(t + copysign(1/2, t)) is exact for binary32 t)
    x = synth.gen_x(512, 11008, seed=33)
    x[0, :32] = 0.0                                        # an all-zero block
    x[1, 32:64] *= np.float32(1e-30)                       # tiny and huge magnitudes
    x[2, 64:96] *= np.float32(1e30)
    x[3, 96:128] = np.float32(-2.5)                        # constant block: every value -127
    blocks = x.reshape(512, -1, 32)
    amax = np.max(np.abs(blocks), axis=2)
    xs = amax / np.float32(127)
    assert xs.dtype == np.float32
    with np.errstate(invalid="ignore", divide="ignore"):
        t = (blocks / xs[..., None]).astype(np.float64)
    assert t.dtype == np.float64
    ref = np.trunc(t + np.copysign(0.5, t))
    ref = np.where(amax[..., None] == 0, 0.0, np.clip(ref, -127, 127)).astype(np.int8).reshape(512, -1)
    xq, xs_o = oracle.quant_act(x)
    assert np.array_equal(xs_o.view(np.uint32), xs.view(np.uint32))
    assert np.array_equal(xq, ref)


# ------------------------------------------------------------ q6_K GEMM

def test_q6k_partials_constant_closed_form():
    # every code q and every activation code xq constant: P16 = 16 (q - 32) xq
    n, k = 2, 256
    q = np.full((n, k), 45, dtype=np.int32)
    ql, qh = oracle.pack_q6k(q)
    sc = np.arange(1, 17, dtype=np.int8)[None, None, :].repeat(n, 0)
    m = oracle.Mat(oracle.Q6_K, n, k, {"ql": ql, "qh": qh, "sc": sc, "d": f16(np.ones((n, 1)))})
    xq = np.full((1, k), -7, dtype=np.int8)
    p16, i32 = oracle.q6k_partials(m, xq, [0, 0], [0, 1])
    assert np.all(p16 == 16 * 13 * -7)
    assert i32[0].tolist() == [(2 * c + 1 + 2 * c + 2) * 16 * 13 * -7 for c in range(8)]


def test_q6k_partials_brute_force_tiny():
    w = synth.gen_weights(synth.FMT_Q6_K, 3, 512, seed=21)
    m = oracle.Mat(oracle.Q6_K, 3, 512, w)
    xq, xs = oracle.quant_act(synth.gen_x(2, 512, seed=21))
    q = oracle.codes(m).astype(np.int64) - 32
    sc = w["sc"].reshape(3, 32).astype(np.int64)
    mm, nn = np.meshgrid(np.arange(2), np.arange(3), indexing="ij")
    p16, i32 = oracle.q6k_partials(m, xq, mm.ravel(), nn.ravel())
    for p, (mi, ni) in enumerate(zip(mm.ravel(), nn.ravel())):
        prod = (q[ni] * xq[mi].astype(np.int64)).reshape(32, 16)
        assert np.array_equal(p16[p], prod.sum(axis=1))
        assert np.array_equal(i32[p], (prod.sum(axis=1) * sc[ni]).reshape(16, 2).sum(axis=1))


def test_q6k_gemm_equals_dense_matmul_of_dequantized_operands():
    # the blocked form sum_s d sum_c xs I32 equals W @ (xs * xq) over the reals
    w = synth.gen_weights(synth.FMT_Q6_K, 6, 768, seed=22)
    m = oracle.Mat(oracle.Q6_K, 6, 768, w)
    x = synth.gen_x(5, 768, seed=22)
    y, b, xq, xs = oracle.q6k_gemm(m, x)
    xhat = np.repeat(xs.astype(np.float64), 32, axis=1) * xq
    W = oracle.dequant(m)
    ref = xhat @ W.T
    assert np.all(np.abs(y - ref) <= 1e-13 * (np.abs(xhat) @ np.abs(W).T))
    assert np.allclose(b, np.abs(xhat) @ np.abs(W).T, rtol=1e-13, atol=0)


def test_q4_0_gemv_q8_equals_dense_matmul_of_dequantized_operands():
    # the blocked integer form sum_b d xs I equals W @ (xs * xq) over the reals
    w = synth.gen_weights(synth.FMT_Q4_0, 7, 320, seed=23)
    m = oracle.Mat(oracle.Q4_0, 7, 320, w)
    x = synth.gen_x(3, 320, seed=23)
    xq, xs = oracle.quant_act(x)
    y, b = oracle.q4_0_gemv_q8(m, xq, xs)
    xhat = np.repeat(xs.astype(np.float64), 32, axis=1) * xq
    W = oracle.dequant(m)
    assert np.all(np.abs(y - xhat @ W.T) <= 1e-13 * (np.abs(xhat) @ np.abs(W).T))
    assert np.allclose(b, np.abs(xhat) @ np.abs(W).T, rtol=1e-13, atol=0)
    # sampled rows are the same numbers as the full call
    ys, bs = oracle.q4_0_gemv_q8(m, xq, xs, rows=[6, 0, 3])
    assert np.array_equal(ys, y[:, [6, 0, 3]]) and np.array_equal(bs, b[:, [6, 0, 3]])


def test_q4_0_gemv_q8_on_exactly_quantizable_activations_is_the_plain_gemv():
    # integer activations whose every 32-block reaches +-127 quantize exactly (xs = 1,
    # xq = x), so the integer form must reproduce the plain double GEMV
    rng = np.random.default_rng(24)
    k = 256
    x = rng.integers(-127, 128, size=(2, k)).astype(np.float32)
    x[:, ::32] = 127.0 * rng.choice([-1, 1], size=(2, k // 32))
    w = synth.gen_weights(synth.FMT_Q4_0, 5, k, seed=24)
    m = oracle.Mat(oracle.Q4_0, 5, k, w)
    xq, xs = oracle.quant_act(x)
    assert np.all(xs == 1.0) and np.array_equal(xq.astype(np.float32), x)
    y, b = oracle.q4_0_gemv_q8(m, xq, xs)
    yr, br = oracle.gemv(m, x)
    assert np.allclose(y, yr, rtol=1e-13, atol=0) and np.allclose(b, br, rtol=1e-13, atol=0)


def test_q4_0_gemv_q8_constant_codes_closed_form():
    # every code c: y = sum_b d_b * xs_b * (c - 8) * sum of the block's xq
    n, k = 3, 128
    xq = np.random.default_rng(25).integers(-127, 128, size=(2, k)).astype(np.int8)
    xs = np.array([[0.5, 0.25, 2.0, 1.0], [1.5, 0.125, 4.0, 0.75]], dtype=np.float32)
    d = np.array([[0x3C00, 0x4000, 0x3800, 0x3C00]] * n, dtype=np.uint16)  # 1, 2, 0.5, 1
    for c in (0, 8, 15):
        qs = oracle.pack_q4_0(np.full((n, k), c, dtype=np.int32))
        m = oracle.Mat(oracle.Q4_0, n, k, {"qs": qs, "d": d})
        y, _ = oracle.q4_0_gemv_q8(m, xq, xs)
        blocks = xq.astype(np.int64).reshape(2, 4, 32).sum(axis=2)
        want = (np.array([1.0, 2.0, 0.5, 1.0]) * xs * (c - 8) * blocks).sum(axis=1)
        assert np.array_equal(y, np.repeat(want[:, None], n, axis=1)), c


def test_moe_gateup_composition():
    gw = synth.gen_weights(synth.FMT_CB4, 8, 256, seed=1, expert=3, matrix=0)
    uw = synth.gen_weights(synth.FMT_CB4, 8, 256, seed=1, expert=3, matrix=1)
    g, u = oracle.Mat(oracle.CB4, 8, 256, gw), oracle.Mat(oracle.CB4, 8, 256, uw)
    x = synth.gen_x(1, 256, synth.DT_BF16, seed=1)
    h, gv, uv, _, _ = oracle.moe_gateup(g, u, x, oracle.BF16)
    xd = synth.bf16_bits_to_f32(x[0]).astype(np.float64)
    G, U = oracle.dequant(g) @ xd, oracle.dequant(u) @ xd
    ref = G / (1 + np.exp(-G)) * U
    assert np.allclose(h, ref, rtol=1e-12, atol=1e-15)
