"""The C-ABI library loads, exports every symbol include/mx.h declares, and
rejects bad arguments on the host with the documented status codes (no GPU
needed: every case here returns before anything is launched)."""
import ctypes
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def mx():
    from microscaling_block_scaled_amd import mx as m
    return m


def header_functions():
    src = open(os.path.join(ROOT, "include", "mx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(mx):
    names = header_functions()
    assert set(names) == set(mx.EXPORTS)
    lib = ctypes.CDLL(mx.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_helpers_match_oracle(mx, oracle):
    for fmt in range(6):
        for rows, cols in [(0, 0), (1, 32), (7, 96), (128, 4096)]:
            assert mx.packed_bytes(fmt, rows, cols) == oracle.packed_bytes(fmt, rows, cols)
            assert mx.scale_bytes(rows, cols) == rows * (cols // 32)
        # a short last block is stored padded to 32 elements
        for rows, cols in [(1, 33), (7, 70), (3, 1), (5, 4095)]:
            assert mx.packed_bytes(fmt, rows, cols) == oracle.packed_bytes(fmt, rows, cols)
            assert mx.packed_bytes(fmt, rows, cols) == mx.packed_bytes(fmt, rows, (cols + 31) // 32 * 32)
            assert mx.scale_bytes(rows, cols) == rows * ((cols + 31) // 32)
    assert mx.packed_bytes(9, 1, 32) == -1
    assert mx.packed_bytes(0, -1, 32) == -1
    assert mx.scale_bytes(-1, 32) == -1
    assert mx.status_str(mx.MX_ERR_SHAPE) == "invalid shape"
    assert mx.version().startswith("mx-gfx950")


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first

# The cases below pass fake device pointers that validation must reject before
# any launch.  Where a GPU is visible they are skipped, so that a case that
# wrongly passed validation could never reach a kernel.
no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0, reason="fake-pointer cases run on CPU only")


def q(mx, x=FAKE, rows=64, cols=64, ld=64, src=1, fmt=0, lay=1, rnd=0, flags=0,
      qr=FAKE, sr=FAKE, qc=FAKE, sc=FAKE, params=True):
    p = mx.QuantParams(src, fmt, lay, rnd, flags, 0, 0, 0)
    return mx.lib.mx_quantize(x, rows, cols, ld, ctypes.byref(p) if params else None,
                              qr, sr, qc, sc, None)


@no_gpu
def test_quantize_validation(mx):
    assert q(mx, params=False) == mx.MX_ERR_ARG
    assert q(mx, src=2) == mx.MX_ERR_ARG
    assert q(mx, fmt=6) == mx.MX_ERR_ARG
    assert q(mx, fmt=-1) == mx.MX_ERR_ARG
    assert q(mx, rnd=2) == mx.MX_ERR_ARG
    assert q(mx, lay=0) == mx.MX_ERR_ARG
    assert q(mx, lay=4) == mx.MX_ERR_ARG
    assert q(mx, flags=2) == mx.MX_ERR_ARG
    assert q(mx, rows=-1) == mx.MX_ERR_ARG
    assert q(mx, ld=32) == mx.MX_ERR_SHAPE
    assert q(mx, cols=48, ld=40) == mx.MX_ERR_SHAPE
    assert q(mx, qr=None) == mx.MX_ERR_ARG
    assert q(mx, lay=2, sc=None) == mx.MX_ERR_ARG
    assert q(mx, x=None) == mx.MX_ERR_ARG
    assert q(mx, x=FAKE + 4) == mx.MX_ERR_ALIGN
    assert q(mx, ld=68) == mx.MX_ERR_ALIGN        # 136-byte bf16 rows
    assert q(mx, src=0, ld=66) == mx.MX_ERR_ALIGN       # 264-byte fp32 rows
    assert q(mx, qr=FAKE + 8) == mx.MX_ERR_ALIGN
    # empty tensors are valid and launch nothing
    assert q(mx, rows=0, x=None) == mx.MX_OK
    assert q(mx, rows=0, cols=0, ld=0, lay=3, x=None) == mx.MX_OK


@no_gpu
def test_dequantize_validation(mx):
    L = mx.lib
    assert L.mx_dequantize(FAKE, FAKE, 7, 4, 32, FAKE, None) == mx.MX_ERR_ARG
    assert L.mx_dequantize(FAKE, FAKE, 0, -4, 32, FAKE, None) == mx.MX_ERR_ARG
    assert L.mx_dequantize(None, FAKE, 0, 4, 32, FAKE, None) == mx.MX_ERR_ARG
    assert L.mx_dequantize(FAKE + 1, FAKE, 0, 4, 32, FAKE, None) == mx.MX_ERR_ALIGN
    assert L.mx_dequantize(FAKE, FAKE, 0, 4, 32, FAKE + 4, None) == mx.MX_ERR_ALIGN
    assert L.mx_dequantize(None, None, 0, 0, 32, None, None) == mx.MX_OK


@no_gpu
def test_gemm_validation(mx):
    L = mx.lib
    g = lambda af=0, bf=0, M=64, N=64, K=64, ldc=64, a=FAKE, b=FAKE, c=FAKE: L.mx_gemm(
        a, FAKE, af, b, FAKE, bf, M, N, K, c, ldc, None)
    assert g(af=6) == mx.MX_ERR_ARG
    assert g(bf=-2) == mx.MX_ERR_ARG
    assert g(af=5) == mx.MX_ERR_UNSUPPORTED
    assert g(bf=5) == mx.MX_ERR_UNSUPPORTED
    assert g(M=-1) == mx.MX_ERR_ARG
    assert g(ldc=63) == mx.MX_ERR_SHAPE
    assert g(c=None) == mx.MX_ERR_ARG
    assert g(a=None) == mx.MX_ERR_ARG
    assert g(a=FAKE + 2) == mx.MX_ERR_ALIGN
    assert g(M=0, c=None) == mx.MX_OK


@no_gpu
def test_gemm_mx_validation(mx):
    L = mx.lib
    g = lambda af=0, bf=0, M=64, N=64, K=512, cf=0, a=FAKE, ascale=FAKE, cq=FAKE, cs=FAKE: \
        L.mx_gemm_mx(a, ascale, af, FAKE, FAKE, bf, M, N, K, cf, cq, cs, None)
    assert g(af=6) == mx.MX_ERR_ARG
    assert g(cf=6) == mx.MX_ERR_ARG
    assert g(cf=-1) == mx.MX_ERR_ARG
    assert g(af=5) == mx.MX_ERR_UNSUPPORTED
    for cf in (2, 3, 5):  # FP6 and INT8 outputs are not fused
        assert g(cf=cf) == mx.MX_ERR_UNSUPPORTED
    assert g(M=-1) == mx.MX_ERR_ARG
    assert g(cq=None) == mx.MX_ERR_ARG
    assert g(cs=None) == mx.MX_ERR_ARG
    assert g(a=None) == mx.MX_ERR_ARG
    assert g(cq=FAKE + 4) == mx.MX_ERR_ALIGN
    assert g(a=FAKE + 2) == mx.MX_ERR_ALIGN
    # outside the staged kernel: refused before any launch
    assert g(K=96) == mx.MX_ERR_UNSUPPORTED
    assert g(K=48) == mx.MX_ERR_UNSUPPORTED   # padded to 64: not a multiple of 512
    assert g(K=0) == mx.MX_ERR_UNSUPPORTED
    assert g(ascale=FAKE + 1) == mx.MX_ERR_UNSUPPORTED
    assert g(M=0, cq=None, cs=None) == mx.MX_OK
    assert g(N=0, cq=None, cs=None) == mx.MX_OK


@no_gpu
def test_gemm_bf16_validation(mx):
    L = mx.lib
    g = lambda af=0, bf=0, M=64, N=64, K=64, ldc=64, a=FAKE, c=FAKE: L.mx_gemm_bf16(
        a, FAKE, af, FAKE, FAKE, bf, M, N, K, c, ldc, None)
    assert g(af=6) == mx.MX_ERR_ARG
    assert g(af=5) == mx.MX_ERR_UNSUPPORTED
    assert g(M=-1) == mx.MX_ERR_ARG
    assert g(ldc=63) == mx.MX_ERR_SHAPE
    assert g(c=None) == mx.MX_ERR_ARG
    assert g(a=None) == mx.MX_ERR_ARG
    assert g(a=FAKE + 2) == mx.MX_ERR_ALIGN
    assert g(c=FAKE + 1) == mx.MX_ERR_ALIGN
    assert g(M=0, c=None) == mx.MX_OK
