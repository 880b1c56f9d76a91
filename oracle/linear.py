"""fp64 oracle for the linear layers around the attention (vitattn_linear).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may use it; the library never imports it.

What it computes is the plain definition of a linear layer with bias and an
optional residual add, as a ViT block applies it before and after the
attention: the fused qkv projection (FluxVLA "Inference acceleration",
section 1; the Pi0 Flash Attention tutorial, section 3.2, feeds the
attention from it) and the output projection with bias and residual (same
FluxVLA page, section 3):

    out[m][n] = sum_k x[m][k] * w[n][k] + bias[n] + residual[m][n]

The 16-bit inputs (bf16 or fp16 bit patterns) are widened exactly to
float64 and the product is numpy's float64 matrix product; nothing is
rounded back to 16 bits.
"""
from __future__ import annotations

import numpy as np


def widen(bits, fmt: str = "bf16") -> np.ndarray:
    """Exact float64 values of 16-bit patterns: bf16 is the top half of an
    IEEE float32, fp16 is IEEE binary16."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    if fmt == "bf16":
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if fmt == "f16":
        return b.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown element format {fmt!r}")


def linear(x, w, bias=None, residual=None, fmt: str = "bf16") -> np.ndarray:
    """x: [M, K] bits, w: [Nout, K] bits, bias: [Nout] bits or None,
    residual: [M, Nout] bits or None.  Returns float64 [M, Nout]."""
    xf = widen(x, fmt)
    wf = widen(w, fmt)
    if xf.ndim != 2 or wf.ndim != 2 or xf.shape[1] != wf.shape[1]:
        raise ValueError("x must be [M, K] and w [Nout, K]")
    out = xf @ wf.T
    if bias is not None:
        out = out + widen(bias, fmt)[None, :]
    if residual is not None:
        out = out + widen(residual, fmt)
    return out


def linear_rows(x, w, bias, residual, rows, fmt: str = "bf16") -> np.ndarray:
    """The rows `rows` (indices into M) of linear(x, w, bias, residual):
    float64 [len(rows), Nout]."""
    rows = np.asarray(rows, dtype=np.int64)
    xr = np.asarray(x)[rows]
    rr = None if residual is None else np.asarray(residual)[rows]
    return linear(xr, w, bias, rr, fmt)
