"""ctypes binding of libvitattn's C ABI (include/vitattn.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  PyTorch supplies device memory and the current HIP stream.
There is no CPU or PyTorch fallback: if the shared library is missing the
import fails.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libvitattn.so")

LAYOUT_SEPARATE = 0  # VITATTN_LAYOUT_SEPARATE_BHND: q, k, v [B,H,N,D]; out [B,H,N,D]
LAYOUT_PACKED = 1    # VITATTN_LAYOUT_PACKED_BN3HD: qkv [B,N,3,H,D]; out [B,N,H,D]

# status codes of include/vitattn.h
OK = 0
ERR_NULL_POINTER = -1
ERR_BAD_SIZE = -2
ERR_UNSUPPORTED_D = -3
ERR_BAD_SCALE = -4
ERR_BAD_LAYOUT = -5
ERR_MISALIGNED = -6
ERR_TOO_LARGE = -7
ERR_LAUNCH = -8
ERR_OVERLAP = -9

EXPORTED = ("vitattn_fwd", "vitattn_strerror", "vitattn_version")


class VitAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"vitattn error {status}: {message}")
        self.status = status


def _load(path: str = LIBRARY):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built: libvitattn has no fallback; build it with "
            "__graft_entry__.build() or vit_self_attention_amd.build.build()")
    lib = ctypes.CDLL(path)
    lib.vitattn_fwd.restype = ctypes.c_int
    lib.vitattn_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.vitattn_strerror.restype = ctypes.c_char_p
    lib.vitattn_strerror.argtypes = [ctypes.c_int]
    lib.vitattn_version.restype = ctypes.c_int
    lib.vitattn_version.argtypes = []
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.vitattn_strerror(int(status)).decode()


def version() -> int:
    return lib.vitattn_version()


def fwd_raw(qkv_or_q: int, k: int | None, v: int | None, out: int, B: int, H: int, N: int,
            D: int, scale: float, layout: int, stream: int | None) -> int:
    """Direct call of vitattn_fwd with raw device addresses; returns the status."""
    return lib.vitattn_fwd(qkv_or_q or None, k or None, v or None, out or None, int(B), int(H),
                           int(N), int(D), float(scale), int(layout), stream or None)


def fwd(q_or_qkv, k=None, v=None, *, out=None, scale: float | None = None, stream=None):
    """O = softmax(scale * Q K^T) V per (image, head), on the GPU.

    Packed layout: `fwd(qkv)` with qkv a bf16 CUDA tensor [B, N, 3, H, D]
    (the fused qkv projection); returns out [B, N, H, D].
    Separate layout: `fwd(q, k, v)` with q, k, v bf16 CUDA tensors
    [B, H, N, D]; returns out [B, H, N, D].

    `scale` defaults to 1/sqrt(D).  `out` may be passed preallocated (same
    device, bf16, contiguous, output shape).  The kernel is enqueued on
    `stream` (a torch.cuda.Stream; default: the current stream) and the call
    returns without waiting.
    """
    import torch

    if (k is None) != (v is None):
        raise ValueError("pass both k and v (separate layout) or neither (packed layout)")
    tensors = [q_or_qkv] + ([k, v] if k is not None else [])
    for t in tensors:
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("inputs must be bfloat16 CUDA tensors")
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
        if t.device != q_or_qkv.device:
            raise ValueError("all tensors must be on the same device")
    if k is None:
        if q_or_qkv.dim() != 5 or q_or_qkv.shape[2] != 3:
            raise ValueError(f"packed qkv must be [B,N,3,H,D], got {tuple(q_or_qkv.shape)}")
        B, N, _, H, D = q_or_qkv.shape
        layout = LAYOUT_PACKED
        out_shape = (B, N, H, D)
    else:
        if q_or_qkv.dim() != 4:
            raise ValueError(f"q must be [B,H,N,D], got {tuple(q_or_qkv.shape)}")
        B, H, N, D = q_or_qkv.shape
        if tuple(k.shape) != (B, H, N, D) or tuple(v.shape) != (B, H, N, D):
            raise ValueError("q, k, v must have the same shape [B,H,N,D]")
        layout = LAYOUT_SEPARATE
        out_shape = (B, H, N, D)
    if out is None:
        out = torch.empty(out_shape, dtype=torch.bfloat16, device=q_or_qkv.device)
    else:
        if (out.dtype != torch.bfloat16 or tuple(out.shape) != out_shape
                or not out.is_contiguous() or out.device != q_or_qkv.device):
            raise ValueError(f"out must be a contiguous bf16 tensor {out_shape} on the input device")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if stream is None:
        stream = torch.cuda.current_stream(q_or_qkv.device)
    rc = fwd_raw(q_or_qkv.data_ptr(), k.data_ptr() if k is not None else None,
                 v.data_ptr() if v is not None else None, out.data_ptr(), B, H, N, D, scale,
                 layout, stream.cuda_stream)
    if rc != OK:
        raise VitAttnError(rc, strerror(rc))
    return out
