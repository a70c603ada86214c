"""CPU oracle for MX quantization and the MX dot product.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline leg
of the benchmark are the only callers; the GPU library never imports, links or
runs anything here, and this package imports nothing from the GPU library.

The arithmetic lives in ``mx_oracle.c`` (plain C, built with gcc into
``liboracle.so``); this module builds it and marshals numpy arrays to it.
Definitions followed (see the C file's header for the passages):
"Microscaling Data Formats for Deep Learning", summary sections 2-4, and the
"Format-Aware Fusion for Fast FP4 Pretraining" abstract (stochastic rounding,
fixed-sign 32-value Hadamard).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2, E2M3, E3M2, E2M1, INT8 = range(6)
FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m3": E2M3, "e3m2": E3M2, "e2m1": E2M1, "int8": INT8}
SRC_F32, SRC_BF16 = 0, 1
RNE, SR = 0, 1
LAYOUT_ROW, LAYOUT_COLT = 1, 2
FLAG_HADAMARD32 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (fp contraction off: the Hadamard step is
    defined as separate fp32 adds and multiplies)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    u64 = ctypes.c_uint64
    lib.mxo_elem_value.restype = ctypes.c_double
    lib.mxo_elem_value.argtypes = [ctypes.c_int, ctypes.c_uint]
    lib.mxo_elem_emax.argtypes = [ctypes.c_int]
    lib.mxo_elem_maxnorm.restype = ctypes.c_double
    lib.mxo_elem_maxnorm.argtypes = [ctypes.c_int]
    lib.mxo_elem_bits.argtypes = [ctypes.c_int]
    lib.mxo_quantize_block.argtypes = [ctypes.c_int, P, ctypes.c_int, P, P, P]
    lib.mxo_philox4x32_10.argtypes = [P, P, P]
    lib.mxo_sr_word.restype = ctypes.c_uint32
    lib.mxo_sr_word.argtypes = [u64, u64, ctypes.c_int, u64]
    lib.mxo_hadamard32.argtypes = [P, ctypes.c_uint32]
    lib.mxo_packed_bytes.restype = i64
    lib.mxo_packed_bytes.argtypes = [ctypes.c_int, i64, i64]
    lib.mxo_quantize.argtypes = [ctypes.c_int, P, i64, i64, i64, ctypes.c_int, ctypes.c_uint,
                                 ctypes.c_int, ctypes.c_uint, u64, u64, ctypes.c_uint32,
                                 P, P, P, P]
    lib.mxo_dequantize.argtypes = [P, P, ctypes.c_int, i64, i64, P]
    lib.mxo_gemm_f64.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int, i64, i64, i64, P, P]
    lib.mxo_gemm_f64_at.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int, i64, i64, i64,
                                    P, P, i64, P, P]
    lib.mxo_set_threads.restype = ctypes.c_int
    lib.mxo_set_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def set_threads(n: int = 0) -> int:
    """OpenMP threads of the whole-tensor functions (0: unchanged); returns
    the count in force."""
    return int(_load().mxo_set_threads(n))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def elem_value(fmt: int, code: int) -> float:
    return _load().mxo_elem_value(fmt, code)


def elem_emax(fmt: int) -> int:
    return _load().mxo_elem_emax(fmt)


def elem_maxnorm(fmt: int) -> float:
    return _load().mxo_elem_maxnorm(fmt)


def elem_bits(fmt: int) -> int:
    return _load().mxo_elem_bits(fmt)


def quantize_block(fmt: int, v, round_mode: int = RNE, rnd=None):
    """One 32-element block -> (scale code, 32 unpacked element codes)."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32).reshape(32))
    codes = np.zeros(32, np.uint8)
    sc = np.zeros(1, np.uint8)
    r = None if rnd is None else np.ascontiguousarray(np.asarray(rnd, dtype=np.uint32).reshape(32))
    _load().mxo_quantize_block(fmt, _ptr(v), round_mode, None if r is None else _ptr(r),
                               _ptr(codes), _ptr(sc))
    return int(sc[0]), codes


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.zeros(4, np.uint32)
    _load().mxo_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_word(seed: int, counter_offset: int, layout_id: int, i: int) -> int:
    return int(_load().mxo_sr_word(seed, counter_offset, layout_id, i))


def hadamard32(x, signs: int = 0):
    v = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(32)).copy()
    _load().mxo_hadamard32(_ptr(v), signs)
    return v


def packed_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(_load().mxo_packed_bytes(fmt, rows, cols))


def quantize(x: np.ndarray, fmt: int, layouts: int = LAYOUT_ROW, round_mode: int = RNE,
             flags: int = 0, seed: int = 0, counter_offset: int = 0, hadamard_signs: int = 0,
             src: int | None = None):
    """Quantize a 2-D array.  ``x`` is float32, or uint16 holding bf16 bit
    patterns.  Returns dict with q_row/s_row and/or q_colt/s_colt (uint8).  A
    blocked dimension that is not a multiple of 32 is quantized as if padded
    with zeros to the next multiple (the outputs keep the padded blocks)."""
    if src is None:
        src = SRC_F32 if x.dtype == np.float32 else SRC_BF16
    want = np.float32 if src == SRC_F32 else np.uint16
    x = np.ascontiguousarray(x, dtype=want)
    rows, cols = x.shape
    out = {}
    q_row = s_row = q_colt = s_colt = None
    if layouts & LAYOUT_ROW:
        q_row = np.zeros((rows, packed_bytes(fmt, 1, cols)), np.uint8)
        s_row = np.zeros((rows, (cols + 31) // 32), np.uint8)
        out["q_row"], out["s_row"] = q_row, s_row
    if layouts & LAYOUT_COLT:
        q_colt = np.zeros((cols, packed_bytes(fmt, 1, rows)), np.uint8)
        s_colt = np.zeros((cols, (rows + 31) // 32), np.uint8)
        out["q_colt"], out["s_colt"] = q_colt, s_colt
    p = lambda a: None if a is None else _ptr(a)
    rc = _load().mxo_quantize(src, _ptr(x), rows, cols, cols, fmt, layouts, round_mode, flags,
                              seed, counter_offset, hadamard_signs, p(q_row), p(s_row),
                              p(q_colt), p(s_colt))
    if rc != 0:
        raise ValueError("oracle quantize rejected its arguments")
    return out


def dequantize(q: np.ndarray, s: np.ndarray, fmt: int, rows: int, cols: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    y = np.zeros((rows, cols), np.float32)
    if _load().mxo_dequantize(_ptr(q), _ptr(s), fmt, rows, cols, _ptr(y)) != 0:
        raise ValueError("oracle dequantize rejected its arguments")
    return y


def gemm_f64(a_q, a_s, a_fmt, b_q, b_s, b_fmt, M, N, K):
    """(C, T): C = deq(A) @ deq(B^T)^T in fp64 and T = sum |a*b| per element."""
    a_q, a_s, b_q, b_s = (np.ascontiguousarray(a, dtype=np.uint8) for a in (a_q, a_s, b_q, b_s))
    c = np.zeros((M, N), np.float64)
    t = np.zeros((M, N), np.float64)
    rc = _load().mxo_gemm_f64(_ptr(a_q), _ptr(a_s), a_fmt, _ptr(b_q), _ptr(b_s), b_fmt,
                              M, N, K, _ptr(c), _ptr(t))
    if rc != 0:
        raise ValueError("oracle gemm rejected its arguments")
    return c, t


def gemm_f64_at(a_q, a_s, a_fmt, b_q, b_s, b_fmt, M, N, K, ms, ns):
    a_q, a_s, b_q, b_s = (np.ascontiguousarray(a, dtype=np.uint8) for a in (a_q, a_s, b_q, b_s))
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    c = np.zeros(len(ms), np.float64)
    t = np.zeros(len(ms), np.float64)
    rc = _load().mxo_gemm_f64_at(_ptr(a_q), _ptr(a_s), a_fmt, _ptr(b_q), _ptr(b_s), b_fmt,
                                 M, N, K, _ptr(ms), _ptr(ns), len(ms), _ptr(c), _ptr(t))
    if rc != 0:
        raise ValueError("oracle gemm_at rejected its arguments")
    return c, t
