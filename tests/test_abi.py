"""The C ABI on the host, with no GPU: the library loads, exports every symbol include/mx.h
declares, and every argument error is reported as a status code before any device work."""
import ctypes
import os
import re

import pytest

import block_scaled_precision_act_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mx.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(mx_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.LIB_PATH):
        from block_scaled_precision_act_amd import build
        build.build()
    return mx.load()


def test_header_declares_the_full_boundary():
    names = _declared()
    assert "mx_act_quant" in names and "mx_act_quant_strided_batched" in names
    assert "mx_act_quant_fp4" in names and "mx_act_quant_fp4_strided_batched" in names
    for k in ("fp8_fp4", "fp8_fp8", "fp4_fp4"):
        for v in ("", "_bias", "_strided_batched", "_bias_strided_batched"):
            assert f"mx_gemm_{k}{v}" in names
    for k in ("fp8_fp4", "fp8_fp8"):
        for v in ("_quant", "_quant_strided_batched"):
            assert f"mx_gemm_{k}{v}" in names
    for k in ("fp8_fp4", "fp8_fp8", "fp4_fp4"):
        for v in ("_bias_residual", "_bias_residual_strided_batched", "_bias_gelu",
                  "_bias_gelu_strided_batched"):
            assert f"mx_gemm_{k}{v}" in names
    for k in ("fp8_fp4", "fp8_fp8", "fp4_fp4"):
        assert f"mx_gemm_{k}_splitk" in names
    assert "mx_gemm_splitk_workspace_size" in names
    assert "mx_gemm_fp8_fp4_splitk_noalloc" in names
    for n in ("mx_quant_e5m2", "mx_quant_e5m2_strided_batched", "mx_quant_transpose_e4m3",
              "mx_quant_transpose_e5m2", "mx_gemm_e5m2_e4m3", "mx_gemm_e5m2_e4m3_strided_batched",
              "mx_gemm_e5m2_e4m3_splitk", "mx_gemm_fp4_fp4_quant",
              "mx_gemm_fp4_fp4_quant_strided_batched"):
        assert n in names
    for k in ("fp8_fp4", "fp8_fp8", "fp4_fp4"):
        for v in ("_bias_gelu_quant", "_bias_gelu_quant_strided_batched"):
            assert f"mx_gemm_{k}{v}" in names
    assert "mx_capability" in names and "mx_status_str" in names
    assert len(names) == 54


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_covers_every_declared_symbol():
    for name in _declared():
        if name == "mx_status_str":
            continue
        assert name in mx._SIGS or hasattr(mx, name), name


def test_status_strings(lib):
    for st in range(0, -8, -1):
        s = mx.status_str(st)
        assert s and s != "unknown status"
    assert mx.status_str(-99) == "unknown status"


def test_capability_without_gpu(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    caps = mx.mx_capability()
    assert caps["status"] == mx.MX_ERR_DEVICE and not caps["available"]
    assert caps["reason"]
    assert lib.mx_capability(None) == mx.MX_ERR_NULL


A16 = 1 << 20          # a fake 16-byte-aligned address: never dereferenced by these calls


def _aq(lib, x=A16, q=A16, s=A16, M=4, K=64):
    return lib.mx_act_quant(x, q, s, M, K, None)


def test_act_quant_argument_errors(lib):
    assert _aq(lib, K=48) == mx.MX_ERR_SHAPE
    assert _aq(lib, K=0) == mx.MX_ERR_SHAPE
    assert _aq(lib, M=-1) == mx.MX_ERR_SHAPE
    assert _aq(lib, M=1 << 26, K=64) == mx.MX_ERR_SHAPE       # 2^32 elements in one matrix
    assert _aq(lib, x=None) == mx.MX_ERR_NULL
    assert _aq(lib, s=None) == mx.MX_ERR_NULL
    assert _aq(lib, x=A16 + 2) == mx.MX_ERR_ALIGN
    assert _aq(lib, q=A16 + 8) == mx.MX_ERR_ALIGN
    assert _aq(lib, x=None, M=0) == mx.MX_OK                 # empty: nothing to do
    sb = lib.mx_act_quant_strided_batched
    assert sb(A16, A16, A16, 4, 64, 2, 256, 0, 8, None) == mx.MX_ERR_STRIDE
    assert sb(A16, A16, A16, 4, 64, 2, 256, 256, 0, None) == mx.MX_ERR_STRIDE
    assert sb(A16, A16, A16, 4, 64, 2, -1, 256, 8, None) == mx.MX_ERR_STRIDE
    assert sb(A16, A16, A16, 4, 64, 2, 257, 256, 8, None) == mx.MX_ERR_ALIGN
    assert sb(A16, A16, A16, 4, 64, 70000, 256, 256, 8, None) == mx.MX_ERR_SHAPE
    assert sb(A16, A16, A16, 4, 64, 0, 256, 256, 8, None) == mx.MX_OK


def test_act_quant_fp4_argument_errors(lib):
    f = lib.mx_act_quant_fp4
    assert f(A16, A16, A16, 4, 48, None) == mx.MX_ERR_SHAPE
    assert f(None, A16, A16, 4, 64, None) == mx.MX_ERR_NULL
    assert f(A16, A16 + 4, A16, 4, 64, None) == mx.MX_ERR_ALIGN
    assert f(None, None, None, 0, 64, None) == mx.MX_OK
    fb = lib.mx_act_quant_fp4_strided_batched
    assert fb(A16, A16, A16, 4, 64, 2, 256, 0, 8, None) == mx.MX_ERR_STRIDE
    assert fb(A16, A16, A16, 4, 64, 2, 256, 136, 8, None) == mx.MX_ERR_ALIGN


def test_act_quant_valid_args_without_gpu_report_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _aq(lib) == mx.MX_ERR_DEVICE


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
def test_gemm_argument_errors(lib, kind):
    g = getattr(lib, f"mx_gemm_{kind}")
    gb = getattr(lib, f"mx_gemm_{kind}_bias")
    gs = getattr(lib, f"mx_gemm_{kind}_strided_batched")
    gbs = getattr(lib, f"mx_gemm_{kind}_bias_strided_batched")
    ok = (A16, A16, A16, A16, A16, 16, 16, 64, None)
    assert g(*ok[:7], 48, None) == mx.MX_ERR_SHAPE
    assert g(*ok[:5], -1, 16, 64, None) == mx.MX_ERR_SHAPE
    assert g(*ok[:5], 1 << 16, 1 << 16, 64, None) == mx.MX_ERR_SHAPE   # M*N >= 2^31
    assert g(None, *ok[1:]) == mx.MX_ERR_NULL
    assert g(*ok[:4], None, *ok[5:]) == mx.MX_ERR_NULL
    assert g(A16 + 4, *ok[1:]) == mx.MX_ERR_ALIGN
    assert g(A16, A16, A16 + 1, *ok[3:]) == mx.MX_ERR_ALIGN
    assert g(A16, A16 + 1, A16, A16 + 3, A16 + 2, 16, 16, 64, None) != mx.MX_ERR_ALIGN
    assert gb(A16, A16, A16, A16, None, A16, 16, 16, 64, None) == mx.MX_ERR_NULL
    assert g(None, None, None, None, None, 0, 16, 64, None) == mx.MX_OK
    assert g(None, None, None, None, None, 16, 0, 64, None) == mx.MX_OK
    args = (A16, A16, A16, A16, A16, 16, 16, 64)
    assert gs(*args, 2, 1024, 32, 1024, 32, 0, None) == mx.MX_ERR_STRIDE      # output stride 0
    assert gs(*args, 2, 1024, 32, 1024, 32, -256, None) == mx.MX_ERR_STRIDE
    assert gs(*args, 2, 1000, 32, 1024, 32, 256, None) == mx.MX_ERR_ALIGN     # A batch not 16B
    assert gs(*args, 0, 1024, 32, 1024, 32, 256, None) == mx.MX_OK
    assert gs(*args, 70000, 1024, 32, 1024, 32, 256, None) == mx.MX_ERR_SHAPE
    bargs = (A16, A16, A16, A16, A16, A16, 16, 16, 64)
    assert gbs(*bargs, 2, 1024, 32, 1024, 32, -1, 256, None) == mx.MX_ERR_STRIDE
    assert gbs(A16, A16, A16, A16, None, A16, 16, 16, 64, 2, 0, 0, 0, 0, 0, 256, None) == \
        mx.MX_ERR_NULL


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
@pytest.mark.parametrize("variant", ["_quant", "_bias_gelu_quant"])
def test_gemm_quant_argument_errors(lib, kind, variant):
    g = getattr(lib, f"mx_gemm_{kind}{variant}")
    gs = getattr(lib, f"mx_gemm_{kind}{variant}_strided_batched")
    # a, a_s, b, b_s, bias (may be NULL), q, q_s, M, N, K
    ok = (A16, A16, A16, A16, None, A16, A16, 16, 64, 64)
    assert g(*ok[:7], 16, 48, 64, None) == mx.MX_ERR_SHAPE        # N not a multiple of 32
    assert g(*ok[:7], 16, 64, 48, None) == mx.MX_ERR_SHAPE        # K not a multiple of 32
    assert g(*ok[:5], None, *ok[6:], None) == mx.MX_ERR_NULL      # q
    assert g(*ok[:6], None, *ok[7:], None) == mx.MX_ERR_NULL      # q_scale
    assert g(*ok[:5], A16 + 8, *ok[6:], None) == mx.MX_ERR_ALIGN  # q not 16-byte aligned
    assert g(*ok[:5], A16, A16 + 1, *ok[7:], None) != mx.MX_ERR_ALIGN
    assert g(None, None, None, None, None, None, None, 0, 64, 64, None) == mx.MX_OK
    # batch, sa, sas, sb, sbs, sbias, sq, sqs
    assert gs(*ok, 2, 1024, 32, 4096, 128, 0, 0, 32, None) == mx.MX_ERR_STRIDE   # q stride 0
    assert gs(*ok, 2, 1024, 32, 4096, 128, 0, 1024, 0, None) == mx.MX_ERR_STRIDE  # q_s stride 0
    assert gs(*ok, 2, 1024, 32, 4096, 128, 0, 1032, 32, None) == mx.MX_ERR_ALIGN  # q batch
    assert gs(*ok, 2, 1024, 32, 4096, 128, -1, 1024, 32, None) == mx.MX_ERR_STRIDE


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
def test_gemm_epilogue_argument_errors(lib, kind):
    gr = getattr(lib, f"mx_gemm_{kind}_bias_residual")
    grs = getattr(lib, f"mx_gemm_{kind}_bias_residual_strided_batched")
    gg = getattr(lib, f"mx_gemm_{kind}_bias_gelu")
    ggs = getattr(lib, f"mx_gemm_{kind}_bias_gelu_strided_batched")
    # a, a_s, b, b_s, bias (may be NULL), residual, c, M, N, K
    ok = (A16, A16, A16, A16, None, A16, A16, 16, 64, 64)
    assert gr(*ok[:5], None, *ok[6:], None) == mx.MX_ERR_NULL        # residual
    assert gr(*ok[:6], None, *ok[7:], None) == mx.MX_ERR_NULL        # c
    assert gr(*ok[:7], 16, 64, 40, None) == mx.MX_ERR_SHAPE          # K not a multiple of 32
    assert gr(None, None, None, None, None, None, None, 16, 0, 64, None) == mx.MX_OK   # empty
    # batch, sa, sas, sb, sbs, sbias, sres, sc
    assert grs(*ok, 2, 1024, 32, 4096, 128, 0, -1, 1024, None) == mx.MX_ERR_STRIDE
    assert grs(*ok, 2, 1024, 32, 4096, 128, 0, 1024, 0, None) == mx.MX_ERR_STRIDE   # c stride 0
    assert grs(*ok, 2, 1024, 32, 4096, 128, 0, 0, 1024, None) != mx.MX_ERR_STRIDE   # broadcast
    og = (A16, A16, A16, A16, None, A16, 16, 64, 64)
    assert gg(*og[:5], None, *og[6:], None) == mx.MX_ERR_NULL        # c
    assert gg(*og[:6], 16, 64, 0, None) == mx.MX_ERR_SHAPE
    assert ggs(*og, 2, 1024, 32, 4096, 128, 0, 0, None) == mx.MX_ERR_STRIDE
    assert ggs(*og, 2, 1032, 32, 4096, 128, 0, 1024, None) == mx.MX_ERR_ALIGN


def test_size_limit_is_enforced(lib):
    # each matrix must hold fewer than 2^31 elements: 65535 x 32768 passes validation, 65536 not
    f = lib.mx_act_quant
    assert f(A16, A16, A16, 65536, 32768, None) == mx.MX_ERR_SHAPE
    g = lib.mx_gemm_fp8_fp4
    assert g(A16, A16, A16, A16, A16, 65536, 64, 32768, None) == mx.MX_ERR_SHAPE
    assert g(A16, A16, A16, A16, A16, 64, 65536, 32768, None) == mx.MX_ERR_SHAPE
    assert g(A16, A16, A16, A16, A16, 65536, 32768, 32, None) == mx.MX_ERR_SHAPE   # output
    assert lib.mx_quant_transpose_e4m3(A16, A16, A16, 65536, 32768, None) == mx.MX_ERR_SHAPE
    import torch
    if not torch.cuda.is_available():
        assert f(A16, A16, A16, 65535, 32768, None) == mx.MX_ERR_DEVICE
        assert g(A16, A16, A16, A16, A16, 65535, 64, 32768, None) == mx.MX_ERR_DEVICE


def test_splitk_workspace_size_plan():
    # 256x256 tiles; two K ranges when there are 65..128 tiles and >= 80 K steps of 64;
    # workspace = a counter and a ready flag per tile (rounded up to 256 B) + one fp32 partial
    # tile per output tile.
    def size(tiles):
        return ((tiles * 8 + 255) // 256) * 256 + tiles * 256 * 256 * 4
    assert mx.mx_gemm_splitk_workspace_size(4096, 2048, 7168) == size(128)
    assert mx.mx_gemm_splitk_workspace_size(2000, 4000, 5152) == size(128)
    assert mx.mx_gemm_splitk_workspace_size(1280, 3328, 5120) == size(65)
    assert mx.mx_gemm_splitk_workspace_size(1280, 3328, 5056) == 0        # 79 K steps
    assert mx.mx_gemm_splitk_workspace_size(2048, 2048, 8192) == 0        # 64 tiles
    assert mx.mx_gemm_splitk_workspace_size(4096, 2304, 8192) == 0        # 144 tiles
    assert mx.mx_gemm_splitk_workspace_size(4096, 7168, 2048) == 0        # 448 tiles
    assert mx.mx_gemm_splitk_workspace_size(64, 64, 48) == 0              # invalid K
    assert mx.mx_gemm_splitk_workspace_size(-1, 64, 2048) == 0
    assert mx.mx_gemm_splitk_workspace_size(41, 1536, 6144) == 0        # 6 tiles


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
def test_gemm_splitk_argument_errors(lib, kind):
    g = getattr(lib, f"mx_gemm_{kind}_splitk")
    need = mx.mx_gemm_splitk_workspace_size(4096, 2048, 7168)
    # a, a_s, b, b_s, bias, c, M, N, K, workspace, workspace_bytes
    base = (A16, A16, A16, A16, None, A16, 4096, 2048, 7168)
    assert g(*base, None, 0, None) == mx.MX_ERR_WORKSPACE
    assert g(*base, A16, need - 1, None) == mx.MX_ERR_WORKSPACE
    assert g(*base, A16 + 16, need, None) == mx.MX_ERR_WORKSPACE          # not 256-B aligned
    assert g(A16, A16, A16, A16, None, None, 4096, 2048, 7168, A16, need, None) == mx.MX_ERR_NULL
    assert g(*base[:8], 7000, A16, need, None) == mx.MX_ERR_SHAPE
    import torch
    if not torch.cuda.is_available():
        assert g(*base, A16, need, None) == mx.MX_ERR_DEVICE
        # a shape that is not split needs no workspace
        assert g(A16, A16, A16, A16, None, A16, 4096, 7168, 2048, None, 0, None) == mx.MX_ERR_DEVICE


def test_backward_operand_argument_errors(lib):
    q5 = lib.mx_quant_e5m2
    assert q5(A16, A16, A16, 4, 48, 1, 7, None) == mx.MX_ERR_SHAPE          # K % 32
    assert q5(None, A16, A16, 4, 64, 0, 0, None) == mx.MX_ERR_NULL
    assert q5(A16 + 2, A16, A16, 4, 64, 0, 0, None) == mx.MX_ERR_ALIGN
    assert q5(None, None, None, 0, 64, 1, 3, None) == mx.MX_OK              # empty
    qb = lib.mx_quant_e5m2_strided_batched
    assert qb(A16, A16, A16, 4, 64, 2, 256, 0, 8, 1, 1, None) == mx.MX_ERR_STRIDE
    for name, extra in (("mx_quant_transpose_e4m3", ()), ("mx_quant_transpose_e5m2", (1, 5))):
        f = getattr(lib, name)
        assert f(A16, A16, A16, 48, 64, *extra, None) == mx.MX_ERR_SHAPE    # R % 32
        assert f(A16, A16, A16, 64, 12, *extra, None) == mx.MX_ERR_SHAPE    # C % 8
        assert f(A16, A16, None, 64, 64, *extra, None) == mx.MX_ERR_NULL
        assert f(A16, A16 + 4, A16, 64, 64, *extra, None) == mx.MX_ERR_ALIGN
        assert f(None, None, None, 0, 64, *extra, None) == mx.MX_OK
        assert f(A16, A16, A16, 1 << 16, 1 << 16, *extra, None) == mx.MX_ERR_SHAPE
    sk = lib.mx_gemm_e5m2_e4m3_splitk
    assert sk(A16, A16, A16, A16, A16, 4096, 2048, 7168, None, 0, None) == mx.MX_ERR_WORKSPACE
    g = lib.mx_gemm_e5m2_e4m3
    assert g(A16, A16, A16, A16, A16, 16, 16, 40, None) == mx.MX_ERR_SHAPE
    assert g(A16, A16, None, A16, A16, 16, 16, 64, None) == mx.MX_ERR_NULL
    import torch
    if not torch.cuda.is_available():
        assert q5(A16, A16, A16, 4, 64, 1, 7, None) == mx.MX_ERR_DEVICE
        assert g(A16, A16, A16, A16, A16, 16, 16, 64, None) == mx.MX_ERR_DEVICE
        assert lib.mx_quant_transpose_e5m2(A16, A16, A16, 64, 64, 0, 0, None) == mx.MX_ERR_DEVICE


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
def test_gemm_epilogue_valid_args_without_gpu_report_device(lib, kind):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    gr = getattr(lib, f"mx_gemm_{kind}_bias_residual")
    gg = getattr(lib, f"mx_gemm_{kind}_bias_gelu")
    assert gr(A16, A16, A16, A16, None, A16, A16, 16, 64, 64, None) == mx.MX_ERR_DEVICE
    assert gg(A16, A16, A16, A16, A16, A16, 16, 64, 64, None) == mx.MX_ERR_DEVICE


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8"])
def test_gemm_quant_valid_args_without_gpu_report_device(lib, kind):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    g = getattr(lib, f"mx_gemm_{kind}_quant")
    assert g(A16, A16, A16, A16, None, A16, A16, 16, 64, 64, None) == mx.MX_ERR_DEVICE


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
def test_gemm_valid_args_without_gpu_report_device(lib, kind):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    g = getattr(lib, f"mx_gemm_{kind}")
    assert g(A16, A16, A16, A16, A16, 16, 16, 64, None) == mx.MX_ERR_DEVICE


def test_binding_fails_loudly_without_library(tmp_path):
    saved = mx._lib
    try:
        mx._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            mx.load(str(tmp_path / "missing.so"))
    finally:
        mx._lib = saved


def test_splitk_noalloc_argument_errors(lib):
    # a, a_s, b, b_s, bias (may be NULL), c, M, N, K: refused on the host before any HIP call
    f = lib.mx_gemm_fp8_fp4_splitk_noalloc
    assert f(A16, A16, A16, A16, None, A16, 16, 64, 48, None) == mx.MX_ERR_SHAPE     # K % 32
    assert f(A16, A16, A16, A16, None, None, 16, 64, 64, None) == mx.MX_ERR_NULL     # c
    assert f(None, A16, A16, A16, None, A16, 16, 64, 64, None) == mx.MX_ERR_NULL     # a
    assert f(A16 + 8, A16, A16, A16, None, A16, 16, 64, 64, None) == mx.MX_ERR_ALIGN
    assert f(None, None, None, None, None, None, 0, 64, 64, None) == mx.MX_OK        # empty
    assert f(A16, A16, A16, A16, None, A16, 65536, 64, 32768, None) == mx.MX_ERR_SHAPE


def test_c_driver_links_and_reports_missing_device(tmp_path):
    # The C program that drives the ABI from C (tests/c_abi) is built and links against the
    # library and the HIP runtime; without a GPU it reports that and exits with status 1.
    import importlib.util
    import shutil
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("mx_c_driver_build",
                                                  os.path.join(here, "c_abi", "build.py"))
    c_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(c_build)
    exe = c_build.build()
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the GPU test runs the program")
    (tmp_path / "cases.txt").write_text("")
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "no gfx950 device" in r.stderr
    assert shutil.which("gcc") or shutil.which("cc")
