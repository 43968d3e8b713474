"""The C ABI without a GPU: the library loads, exports every declared symbol, and
the host-side validation and size queries behave as include/qmv.h states."""
import ctypes as C
import os
import re

import pytest

import bit_weight_quantized_dequant_amd as qmv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qm[mv]_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = qmv.lib()
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(L, name), name
    assert qmv.lib().qmv_version().decode().startswith("qmv")


def test_plane_bytes_match_the_format_definitions():
    # q6_K: 210 bytes per 256 weights; 256 x 1024 -> 215,040 B
    assert qmv.weight_bytes(qmv.Q6_K, 256, 1024) == 215040
    assert qmv.weight_bytes(qmv.Q6_K, 1, 256) == 210
    # q4_0: 18 bytes per 32 weights
    assert qmv.weight_bytes(qmv.Q4_0, 4096, 4096) == 9437184
    assert qmv.weight_bytes(qmv.Q4_0, 11008, 4096) == 25362432
    assert qmv.weight_bytes(qmv.Q4_0, 1, 32) == 18
    # 4-bit codebook: 0.75 byte per weight
    assert qmv.weight_bytes(qmv.CB4, 2048, 7168) == 11010048
    # 2-bit additive: 2 bytes per 8 weights + 2 B per row + 8 KiB of codebooks
    assert qmv.plane_bytes(qmv.AQ2X8, 14336, 4096, "codes") == 14680064
    assert qmv.weight_bytes(qmv.AQ2X8, 14336, 4096) == 14680064 + 2 * 14336 + 8192
    # 8-bit codebook: one byte per weight + 512 B of codebook per row
    assert qmv.weight_bytes(qmv.CB8, 2048, 7168) == 2048 * 7168 + 2048 * 512
    assert qmv.plane_bytes(qmv.CB8, 3, 64, "codes") == 192
    # 3-bit additive: 3 bytes per 8 weights + 2 B per row + 12 KiB of codebooks
    assert qmv.plane_bytes(qmv.AQ3X8, 14336, 4096, "codes") == 14336 * 512 * 3
    assert qmv.weight_bytes(qmv.AQ3X8, 14336, 4096) == 14336 * 512 * 3 + 2 * 14336 + 12288
    # the 8-bit codebook has no block: any k has a size, but its kernels take k % 64 == 0
    assert qmv.weight_bytes(qmv.CB8, 4, 96) == 4 * 96 + 4 * 512
    assert qmv.validate(_fake(qmv.CB8, 4, 96), 1, qmv.F32) == -2
    assert qmv.validate(_fake(qmv.CB8, 4, 48), 1, qmv.F32) == -2
    assert qmv.plane_bytes(qmv.Q4_0, 4, 32, "codebook") == 0
    assert qmv.weight_bytes(qmv.Q6_K, 4, 100) == -2
    assert qmv.weight_bytes(9, 4, 256) == -3


def _fake(fmt, n, k, **over):
    base = 1 << 20
    planes = {name: base + 4096 * i for i, name in enumerate(qmv.PLANES[fmt])}
    planes.update(over)
    return qmv.QWeights(fmt, n, k, planes)


@pytest.mark.parametrize("fmt,k", [(qmv.Q4_0, 64), (qmv.Q6_K, 512), (qmv.CB4, 256), (qmv.AQ2X8, 16),
                                   (qmv.CB8, 128), (qmv.AQ3X8, 24)])
def test_validate_accepts_well_formed_descriptors(fmt, k):
    assert qmv.validate(_fake(fmt, 8, k), 1, qmv.F32) == 0
    assert qmv.validate(_fake(fmt, 8, k), 8, qmv.BF16) == 0


def test_validate_error_codes():
    L = qmv.lib()
    assert L.qmv_validate(None, 1, 0) == -1
    assert qmv.validate(_fake(qmv.Q4_0, 8, 48)) == -2          # k not a multiple of 32
    assert qmv.validate(_fake(qmv.Q4_0, 0, 64)) == -2          # n <= 0
    assert qmv.validate(_fake(qmv.Q6_K, 8, 128)) == -2         # k not a multiple of 256
    w = _fake(qmv.Q4_0, 8, 64)
    w._s.fmt = 7
    assert qmv.validate(w) == -3
    assert qmv.validate(_fake(qmv.Q4_0, 8, 64), 1, 5) == -4
    assert qmv.validate(_fake(qmv.Q4_0, 8, 64, d=(1 << 20) + 8)) == -5
    assert qmv.validate(_fake(qmv.Q6_K, 8, 256, qh=0)) == -1
    assert qmv.validate(_fake(qmv.CB8, 8, 128, cb=0)) == -1
    assert qmv.validate(_fake(qmv.AQ3X8, 8, 24, s=0)) == -1
    assert qmv.validate(_fake(qmv.AQ3X8, 8, 20)) == -2         # k not a multiple of 8
    assert qmv.validate(_fake(qmv.Q4_0, 8, 64), 0) == -6
    assert qmv.validate(_fake(qmv.Q4_0, 8, 64), 9) == -6
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert qmv.strerror(code) and qmv.strerror(code) != "unknown status"


def test_calls_reject_bad_arguments_before_any_gpu_work():
    L = qmv.lib()
    w = _fake(qmv.Q4_0, 8, 64)
    assert L.qmv_gemv(w.ref, 1, None, 0, 1 << 20, None) == -1
    assert L.qmv_gemv(w.ref, 1, (1 << 20) + 4, 0, 1 << 20, None) == -5
    assert L.qmm_gemm(w.ref, 4, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None) == -3   # q4_0 has no GEMM
    q6 = _fake(qmv.Q6_K, 8, 256)
    need = L.qmm_workspace_bytes(q6.ref, 4)
    # the GEMM's activation layout pads the tokens to its 128-token tile: xq 128 x 256 int8,
    # then xs fp32 [256 / 32][128]
    assert need == 128 * 256 + 8 * 128 * 4
    assert L.qmm_workspace_bytes(q6.ref, 129) == 256 * 256 + 8 * 256 * 4
    assert L.qmm_gemm(q6.ref, 4, 1 << 20, 1 << 20, 1 << 20, need - 1, None) == -7
    assert L.qmm_gemm_ws(q6.ref, 4, 1 << 20, need - 1, 1 << 20, None) == -7
    assert L.qmm_gemm_ws(q6.ref, 4, (1 << 20) + 16, need, 1 << 20, None) == -5   # ws not 256-aligned
    assert L.qmm_gemm_ws(q6.ref, 4, 1 << 20, need, None, None) == -1
    assert L.qmm_quant_act(1 << 20, 2, 48, 1 << 20, 1 << 20, None) == -2
    assert L.qmv_moe_ffn(None, None, None, 1, None, 1, None, 0, None, None, None) == -1
    g, u, d = _fake(qmv.CB4, 256, 512), _fake(qmv.CB4, 256, 512), _fake(qmv.CB4, 512, 256)
    ga = _fake(qmv.AQ2X8, 256, 512)
    args = (1, 1 << 20, 1, 1 << 20, 0, 1 << 20, 1 << 20, None)
    assert L.qmv_moe_ffn(ga.ref, u.ref, d.ref, *args) == -3        # CB4 experts only
    assert L.qmv_moe_ffn(g.ref, u.ref, _fake(qmv.CB4, 512, 128).ref, *args) == -2  # down k != d_ff


def test_plane_calls_check_arguments_before_any_gpu_work(monkeypatch):
    L = qmv.lib()
    q6 = _fake(qmv.Q6_K, 8, 512)
    # 2 bytes per weight in whole 32-row groups (fragment order)
    assert qmv.plane_bytes_of(q6) == 2 * 32 * 512
    assert qmv.plane_bytes_of(_fake(qmv.Q6_K, 33, 256)) == 2 * 64 * 256
    assert qmv.plane_bytes_of(_fake(qmv.CB4, 8, 512)) == -3        # only q6_K has planes
    assert qmv.plane_bytes_of(_fake(qmv.Q6_K, 8, 300)) == -2
    assert L.qmm_plane_bytes(None) == -1
    base = 1 << 24
    assert L.qmm_register_plane(q6.ref, None, 32768, None) == -1
    assert L.qmm_register_plane(q6.ref, base, 32767, None) == -7     # too small
    assert L.qmm_register_plane(q6.ref, base + 16, 32768, None) == -5  # not 256-byte aligned
    assert L.qmm_register_plane(_fake(qmv.AQ2X8, 8, 512).ref, base, 1 << 20, None) == -3
    # explicit opt-out: nothing is written or recorded, and no GPU work is issued
    monkeypatch.setenv("QMV_Q6K_EXP", "0")
    assert L.qmm_register_plane(q6.ref, base, 32768, None) == 0
    assert qmv.last_path() == "plane.q6k(exp=off)"
    assert L.qmm_unregister_plane(q6.ref) == 0
    assert L.qmm_unregister_plane(None) == -1


def test_binding_rejects_bad_tensor_arguments():
    # the C ABI sees only addresses, so the binding checks dtype, device, layout and shape
    import torch
    x = torch.zeros(4, 64, dtype=torch.float64)
    with pytest.raises(TypeError):
        qmv._need(x, (torch.float32,), (4, 64), "x")
    with pytest.raises(ValueError, match="device"):
        qmv._need(x.float(), (torch.float32,), (4, 64), "x")
    qmv._need(1 << 20, (torch.float32,), (4, 64), "x")      # raw addresses pass unchecked
    with pytest.raises(ValueError, match="device"):
        qmv.QWeights(qmv.Q4_0, 8, 64, {"qs": torch.zeros(256, dtype=torch.uint8),
                                        "d": 1 << 20})


@pytest.mark.parametrize("fmt,n,k", [(qmv.Q4_0, 5, 96), (qmv.Q6_K, 3, 512), (qmv.CB4, 4, 256),
                                     (qmv.AQ2X8, 3, 64), (qmv.CB8, 2, 128), (qmv.AQ3X8, 3, 48)])
def test_synthetic_planes_have_the_library_sizes(fmt, n, k):
    # the binding refuses planes shorter than the library's size for them; the generator's
    # planes are exactly that size
    import synth
    w = synth.gen_weights(fmt, n, k, seed=1)
    for name, field in qmv.PLANES[fmt].items():
        assert w[name].nbytes == qmv.plane_bytes(fmt, n, k, field), name


def test_gemv_q8_argument_errors():
    # checked on the host before any HIP call
    L = qmv.lib()
    nz = 1 << 20
    assert L.qmv_gemv_q8(_fake(qmv.CB4, 8, 256).ref, 1, nz, nz, nz, None) == -3    # q4_0 and q6_K only
    assert L.qmv_gemv_q8(_fake(qmv.Q6_K, 8, 16384 + 256).ref, 1, nz, nz, nz, None) == -9
    assert L.qmv_gemv_q8(_fake(qmv.Q4_0, 8, 64).ref, 1, None, nz, nz, None) == -1
    assert L.qmv_gemv_q8(_fake(qmv.Q4_0, 8, 64).ref, 9, nz, nz, nz, None) == -6    # batch > 8
    assert L.qmv_gemv_q8(_fake(qmv.Q4_0, 8, 64).ref, 1, nz + 8, nz, nz, None) == -5
    assert L.qmv_gemv_q8(_fake(qmv.Q4_0, 8, 16384 + 32).ref, 1, nz, nz, nz, None) == -9


def test_read_ceiling_argument_errors():
    L = qmv.lib()
    nz = 1 << 20
    assert L.qmv_read_ceiling(None, 64, nz, None) == -1
    assert L.qmv_read_ceiling(nz, 64, None, None) == -1
    assert L.qmv_read_ceiling(nz, 0, nz, None) == -2
    assert L.qmv_read_ceiling(nz, 40, nz, None) == -2
    assert L.qmv_read_ceiling(nz + 8, 64, nz, None) == -5
    assert L.qmv_read_ceiling(nz, 64, nz + 2, None) == -5


def test_bench_refuses_more_than_one_gpu():
    # one GPU only: the bench says so and exits before touching a device
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)


def test_gemm_noalloc_argument_errors_before_any_gpu_work():
    # the no-allocation GEMM checks everything on the host before it looks up its scratch
    L = qmv.lib()
    nz = 1 << 20
    assert L.qmm_gemm_noalloc(None, 4, nz, nz, None) == -1
    assert L.qmm_gemm_noalloc(_fake(qmv.Q4_0, 8, 256).ref, 4, nz, nz, None) == -3   # q6_K only
    assert L.qmm_gemm_noalloc(_fake(qmv.Q6_K, 8, 300).ref, 4, nz, nz, None) == -2   # k % 256
    assert L.qmm_gemm_noalloc(_fake(qmv.Q6_K, 8, 256).ref, 0, nz, nz, None) == -6
    assert L.qmm_gemm_noalloc(_fake(qmv.Q6_K, 8, 256).ref, 4, None, nz, None) == -1
    assert L.qmm_gemm_noalloc(_fake(qmv.Q6_K, 8, 256).ref, 4, nz + 4, nz, None) == -5
    # beyond the 16 MiB scratch: 512 tokens of k = 29184 need 16,809,984 bytes
    assert qmv.workspace_bytes(_fake(qmv.Q6_K, 8, 29184), 512) > 16 * 1024 * 1024
    assert L.qmm_gemm_noalloc(_fake(qmv.Q6_K, 8, 29184).ref, 512, nz, nz, None) == -9
    assert qmv.workspace_bytes(_fake(qmv.Q6_K, 8, 28928), 512) <= 16 * 1024 * 1024


def test_gemv_ws_sizes_and_argument_errors_before_any_gpu_work():
    # the lookup-table GEMV's workspace: one fp32 partial per k-slice (256 weights for the
    # 2-bit code, 128 for the 3-bit one) and row
    L = qmv.lib()
    nz = 1 << 20
    a2, a3 = _fake(qmv.AQ2X8, 14336, 4096), _fake(qmv.AQ3X8, 14336, 4096)
    assert qmv.gemv_workspace_bytes(a2, 1) == 14336 * 16 * 4
    assert qmv.gemv_workspace_bytes(a3, 1) == 14336 * 32 * 4
    assert qmv.gemv_workspace_bytes(a2, 4) == 0                          # batch 1 only
    assert qmv.gemv_workspace_bytes(_fake(qmv.AQ2X8, 8, 128 * 3), 1) == 0  # k % 256
    assert qmv.gemv_workspace_bytes(_fake(qmv.AQ3X8, 8, 128 * 3), 1) == 8 * 3 * 4
    assert qmv.gemv_workspace_bytes(_fake(qmv.Q4_0, 8, 256), 1) == 0
    assert L.qmv_gemv_workspace_bytes(None, 1) == -1
    assert L.qmv_gemv_workspace_bytes(a2.ref, 0) == -6
    assert L.qmv_gemv_workspace_bytes(_fake(qmv.AQ2X8, 8, 12).ref, 1) == -2
    need = qmv.gemv_workspace_bytes(a2, 1)
    assert L.qmv_gemv_ws(a2.ref, 1, nz, 0, nz, None, need, None) == -7
    assert L.qmv_gemv_ws(a2.ref, 1, nz, 0, nz, nz, need - 1, None) == -7
    assert L.qmv_gemv_ws(a2.ref, 1, nz, 0, nz, nz + 4, need, None) == -5   # ws not 16-byte aligned
    assert L.qmv_gemv_ws(a2.ref, 1, nz + 4, 0, nz, nz, need, None) == -5
    assert L.qmv_gemv_ws(a2.ref, 1, None, 0, nz, nz, need, None) == -1
    assert L.qmv_gemv_ws(a2.ref, 1, nz, 7, nz, nz, need, None) == -4
    assert L.qmv_gemv_ws(a2.ref, 9, nz, 0, nz, nz, need, None) == -6
