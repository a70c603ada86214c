"""ctypes binding of libmx.so (include/mx.h): argument marshalling only.

Every step of the MX path runs in the library's HIP kernels; torch only
provides device memory and the current HIP stream.  Importing this module
without a built library raises immediately: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmx.so")

E4M3, E5M2, E2M3, E3M2, E2M1, INT8 = range(6)
FMT_NAMES = ("e4m3", "e5m2", "e2m3", "e3m2", "e2m1", "int8")
FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m3": E2M3, "e3m2": E3M2, "e2m1": E2M1, "int8": INT8}
BITS = {E4M3: 8, E5M2: 8, E2M3: 6, E3M2: 6, E2M1: 4, INT8: 8}
SRC_F32, SRC_BF16 = 0, 1
RNE, SR = 0, 1
LAYOUT_ROW, LAYOUT_COLT = 1, 2
FLAG_HADAMARD32 = 1
MX_OK, MX_ERR_ARG, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_UNSUPPORTED, MX_ERR_HIP = 0, -1, -2, -3, -4, -5


class QuantParams(ctypes.Structure):
    _fields_ = [("src", ctypes.c_int32), ("fmt", ctypes.c_int32), ("layouts", ctypes.c_uint32),
                ("round", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("hadamard_signs", ctypes.c_uint32), ("seed", ctypes.c_uint64),
                ("counter_offset", ctypes.c_uint64)]


class MXError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run microscaling_block_scaled_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.mx_quantize.restype = ctypes.c_int
    lib.mx_quantize.argtypes = [P, i64, i64, i64, ctypes.POINTER(QuantParams), P, P, P, P, P]
    lib.mx_dequantize.restype = ctypes.c_int
    lib.mx_dequantize.argtypes = [P, P, i32, i64, i64, P, P]
    lib.mx_gemm.restype = ctypes.c_int
    lib.mx_gemm.argtypes = [P, P, i32, P, P, i32, i64, i64, i64, P, i64, P]
    lib.mx_gemm_bf16.restype = ctypes.c_int
    lib.mx_gemm_bf16.argtypes = [P, P, i32, P, P, i32, i64, i64, i64, P, i64, P]
    lib.mx_gemm_mx.restype = ctypes.c_int
    lib.mx_gemm_mx.argtypes = [P, P, i32, P, P, i32, i64, i64, i64, i32, P, P, P]
    lib.mx_packed_bytes.restype = i64
    lib.mx_packed_bytes.argtypes = [i32, i64, i64]
    lib.mx_scale_bytes.restype = i64
    lib.mx_scale_bytes.argtypes = [i64, i64]
    lib.mx_status_str.restype = ctypes.c_char_p
    lib.mx_status_str.argtypes = [ctypes.c_int]
    lib.mx_version.restype = ctypes.c_char_p
    lib.mx_version.argtypes = []
    return lib


lib = _load()

# every symbol include/mx.h declares
EXPORTS = ("mx_quantize", "mx_dequantize", "mx_gemm", "mx_gemm_bf16", "mx_gemm_mx",
           "mx_packed_bytes", "mx_scale_bytes", "mx_status_str", "mx_version")


def status_str(status: int) -> str:
    return lib.mx_status_str(status).decode()


def version() -> str:
    return lib.mx_version().decode()


def packed_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(lib.mx_packed_bytes(fmt, rows, cols))


def scale_bytes(rows: int, cols: int) -> int:
    return int(lib.mx_scale_bytes(rows, cols))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != MX_OK:
        raise MXError(status, what)


def quantize(x: torch.Tensor, fmt: int, layouts: int = LAYOUT_ROW, round_mode: int = RNE,
             hadamard: bool = False, hadamard_signs: int = 0, seed: int = 0,
             counter_offset: int = 0, out: dict | None = None, stream=None) -> dict:
    """MX-quantize a 2-D fp32/bf16 device tensor.  Returns uint8 device tensors
    q_row [rows, packed cols], s_row [rows, blocks of cols] and/or q_colt [cols,
    packed rows], s_colt [cols, blocks of rows]; a short last block is padded
    with zeros to 32 elements.  ``out`` may supply them preallocated."""
    if x.dim() != 2 or x.dtype not in (torch.float32, torch.bfloat16) or not x.is_cuda:
        raise ValueError("x must be a 2-D fp32/bf16 CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    rows, cols = x.shape
    src = SRC_F32 if x.dtype == torch.float32 else SRC_BF16
    o = dict(out or {})
    dev = x.device
    if layouts & LAYOUT_ROW and "q_row" not in o:
        o["q_row"] = torch.empty((rows, packed_bytes(fmt, 1, cols)), dtype=torch.uint8, device=dev)
        o["s_row"] = torch.empty((rows, scale_bytes(1, cols)), dtype=torch.uint8, device=dev)
    if layouts & LAYOUT_COLT and "q_colt" not in o:
        o["q_colt"] = torch.empty((cols, packed_bytes(fmt, 1, rows)), dtype=torch.uint8, device=dev)
        o["s_colt"] = torch.empty((cols, scale_bytes(1, rows)), dtype=torch.uint8, device=dev)
    p = QuantParams(src, fmt, layouts, round_mode, FLAG_HADAMARD32 if hadamard else 0,
                    hadamard_signs & 0xFFFFFFFF, seed, counter_offset)
    st = lib.mx_quantize(_ptr(x), rows, cols, x.stride(0), ctypes.byref(p),
                         _ptr(o.get("q_row")) if layouts & LAYOUT_ROW else None,
                         _ptr(o.get("s_row")) if layouts & LAYOUT_ROW else None,
                         _ptr(o.get("q_colt")) if layouts & LAYOUT_COLT else None,
                         _ptr(o.get("s_colt")) if layouts & LAYOUT_COLT else None,
                         _stream(stream))
    _check(st, "mx_quantize")
    return o


def dequantize(q: torch.Tensor, s: torch.Tensor, fmt: int, rows: int, cols: int,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    y = out if out is not None else torch.empty((rows, cols), dtype=torch.float32, device=q.device)
    _check(lib.mx_dequantize(_ptr(q), _ptr(s), fmt, rows, cols, _ptr(y), _stream(stream)),
           "mx_dequantize")
    return y


def gemm(a_q: torch.Tensor, a_s: torch.Tensor, a_fmt: int, b_q: torch.Tensor, b_s: torch.Tensor,
         b_fmt: int, M: int, N: int, K: int, c: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """C[M, N] fp32 = A[M, K] (row-wise MX) x B where B is given as B^T[N, K]
    (row-wise MX)."""
    if c is None:
        c = torch.empty((M, N), dtype=torch.float32, device=a_q.device)
    _check(lib.mx_gemm(_ptr(a_q), _ptr(a_s), a_fmt, _ptr(b_q), _ptr(b_s), b_fmt, M, N, K,
                       _ptr(c), c.stride(0), _stream(stream)), "mx_gemm")
    return c


def gemm_bf16(a_q: torch.Tensor, a_s: torch.Tensor, a_fmt: int, b_q: torch.Tensor,
              b_s: torch.Tensor, b_fmt: int, M: int, N: int, K: int,
              c: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """``gemm`` with C rounded to bf16 (nearest even) in the kernel."""
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    if c.dtype != torch.bfloat16 or (c.dim() == 2 and c.shape[0] > 0 and c.stride(1) != 1):
        raise ValueError("c must be a bf16 tensor with unit column stride")
    _check(lib.mx_gemm_bf16(_ptr(a_q), _ptr(a_s), a_fmt, _ptr(b_q), _ptr(b_s), b_fmt, M, N, K,
                            _ptr(c), c.stride(0), _stream(stream)), "mx_gemm_bf16")
    return c


def gemm_mx(a_q: torch.Tensor, a_s: torch.Tensor, a_fmt: int, b_q: torch.Tensor,
            b_s: torch.Tensor, b_fmt: int, M: int, N: int, K: int, c_fmt: int,
            out: dict | None = None, stream=None) -> dict:
    """The product of ``gemm`` quantized row-wise (blocks of 32 along N, round to
    nearest even) into format ``c_fmt`` inside the GEMM.  Returns uint8 device
    tensors q_row [M, packed N] and s_row [M, blocks of N] (a short last block
    padded); ``out`` may supply them preallocated."""
    o = dict(out or {})
    dev = a_q.device
    if "q_row" not in o:
        o["q_row"] = torch.empty((M, packed_bytes(c_fmt, 1, N)), dtype=torch.uint8, device=dev)
        o["s_row"] = torch.empty((M, scale_bytes(1, N)), dtype=torch.uint8, device=dev)
    _check(lib.mx_gemm_mx(_ptr(a_q), _ptr(a_s), a_fmt, _ptr(b_q), _ptr(b_s), b_fmt, M, N, K,
                          c_fmt, _ptr(o["q_row"]), _ptr(o["s_row"]), _stream(stream)),
           "mx_gemm_mx")
    return o
