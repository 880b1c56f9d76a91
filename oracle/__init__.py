"""fp64 CPU oracle for the vision-encoder self-attention forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The library
(`vit_self_attention_amd`) never imports it and has no CPU fallback.

The arithmetic lives in `vitattn_oracle.c` (plain C, fp64, OpenMP over
(image, head) pairs); this module only builds it with gcc and marshals numpy
arrays through ctypes.  What it computes is the plain definition of softmax
attention, O = softmax(scale * Q K^T) V over all tokens of each (image, head),
which the Pi0 Flash Attention tutorial (sections 1 and 4.2) says the fast
kernel reproduces without changing the model's output.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "vitattn_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

LAYOUT_SEPARATE = 0
LAYOUT_PACKED = 1
FORMATS = {"bf16": 0, "f16": 1}  # element formats of the 16-bit inputs

_lib = None


def build(source: str = SOURCE, library: str = LIBRARY) -> str:
    """Compile the C oracle into a shared library with gcc and OpenMP."""
    tmp = library + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, library)
    return library


def _bind(lib):
    u16p = ctypes.POINTER(ctypes.c_uint16)
    dp = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_attention_fmt.restype = ctypes.c_int
    lib.oracle_attention_fmt.argtypes = [u16p, u16p, u16p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_double, dp, dp]
    lib.oracle_attention_rows_fmt.restype = ctypes.c_int
    lib.oracle_attention_rows_fmt.argtypes = [u16p, u16p, u16p, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_double, i64p, ctypes.c_int64,
                                              dp]
    lib.oracle_widen.restype = ctypes.c_double
    lib.oracle_widen.argtypes = [ctypes.c_uint, ctypes.c_int]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [u16p, u16p, u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp]
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [u16p, u16p, u16p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double, i64p, ctypes.c_int64, dp]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    return lib


def load(path: str | None = None):
    """Load the built oracle library (building it first if nothing is built)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        _lib = _bind(ctypes.CDLL(LIBRARY))
    return _lib


def _u16(a):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _check_shapes(qkv_or_q, k, v, layout, B, H, N, D):
    if layout == LAYOUT_PACKED:
        if tuple(qkv_or_q.shape) != (B, N, 3, H, D):
            raise ValueError(f"packed input must be [B,N,3,H,D]={(B, N, 3, H, D)}, got {qkv_or_q.shape}")
    elif layout == LAYOUT_SEPARATE:
        for t in (qkv_or_q, k, v):
            if t is None or tuple(t.shape) != (B, H, N, D):
                raise ValueError(f"separate inputs must be [B,H,N,D]={(B, H, N, D)}")
    else:
        raise ValueError(f"unknown layout {layout}")


def _fmt(fmt: str) -> int:
    if fmt not in FORMATS:
        raise ValueError(f"unknown element format {fmt!r}")
    return FORMATS[fmt]


def widen(bits: int, fmt: str = "bf16", lib=None) -> float:
    """The exact value of one 16-bit pattern in element format `fmt`."""
    return (lib or load()).oracle_widen(int(bits), _fmt(fmt))


def attention(qkv_or_q, k, v, layout: int, B: int, H: int, N: int, D: int, scale: float,
              want_probs: bool = False, lib=None, fmt: str = "bf16"):
    """O = softmax(scale Q K^T) V for every (image, head), in fp64.

    Inputs are 16-bit patterns (uint16) in `layout`, bf16 or, with
    fmt="f16", IEEE fp16.  Returns O as float64
    [B, N, H, D] (logical order, whatever the input layout), and P as float64
    [B, H, N, N] too when `want_probs`.
    """
    lib = lib or load()
    _check_shapes(qkv_or_q, k, v, layout, B, H, N, D)
    a, ap = _u16(qkv_or_q)
    kk, kp = _u16(k)
    vv, vp = _u16(v)
    out = np.zeros((B, N, H, D), dtype=np.float64)
    probs = np.zeros((B, H, N, N), dtype=np.float64) if want_probs else None
    rc = lib.oracle_attention_fmt(ap, kp, vp, layout, _fmt(fmt), B, H, N, D, float(scale),
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                  probs.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
                                  if want_probs else None)
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed with {rc}")
    return (out, probs) if want_probs else out


def attention_rows(qkv_or_q, k, v, layout: int, B: int, H: int, N: int, D: int, scale: float,
                   rows, lib=None, fmt: str = "bf16"):
    """O[b, i, h, :] in fp64 for each (b, h, i) triple of `rows` ([R, 3] ints).

    Returns float64 [R, D].
    """
    lib = lib or load()
    _check_shapes(qkv_or_q, k, v, layout, B, H, N, D)
    a, ap = _u16(qkv_or_q)
    kk, kp = _u16(k)
    vv, vp = _u16(v)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    out = np.zeros((r.shape[0], D), dtype=np.float64)
    rc = lib.oracle_attention_rows_fmt(ap, kp, vp, layout, _fmt(fmt), B, H, N, D, float(scale),
                                       r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                       r.shape[0],
                                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_rows failed with {rc}")
    return out


def max_threads(lib=None) -> int:
    return (lib or load()).oracle_max_threads()


def set_threads(n: int, lib=None) -> None:
    (lib or load()).oracle_set_threads(int(n))
