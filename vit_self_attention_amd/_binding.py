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
DTYPE_FP16 = 16      # VITATTN_DTYPE_FP16, OR-ed into the layout: fp16 instead of bf16

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
ERR_GRAPH = -10
ERR_UNSUPPORTED_SHAPE = -11

EXPORTED = ("vitattn_fwd", "vitattn_fwd_shape", "vitattn_linear", "vitattn_plan_create", "vitattn_plan_destroy",
            "vitattn_plan_launch", "vitattn_strerror", "vitattn_version")


class VitAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"vitattn error {status}: {message}")
        self.status = status


def _load(path: str = LIBRARY):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built: libvitattn has no fallback; build it with "
            "__graft_entry__.build() or python vit_self_attention_amd/build.py")
    lib = ctypes.CDLL(path)
    lib.vitattn_fwd.restype = ctypes.c_int
    lib.vitattn_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    ptrs = ctypes.POINTER(ctypes.c_void_p)
    lib.vitattn_plan_create.restype = ctypes.c_int
    lib.vitattn_plan_create.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ptrs, ptrs, ptrs,
                                        ptrs, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_int]
    lib.vitattn_plan_launch.restype = ctypes.c_int
    lib.vitattn_plan_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.vitattn_plan_destroy.restype = ctypes.c_int
    lib.vitattn_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.vitattn_linear.restype = ctypes.c_int
    lib.vitattn_linear.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    ip = ctypes.POINTER(ctypes.c_int)
    lib.vitattn_fwd_shape.restype = ctypes.c_int
    lib.vitattn_fwd_shape.argtypes = [ctypes.c_int] * 5 + [ip] * 4
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


def fwd_shape(B: int, H: int, N: int, D: int, layout: int = LAYOUT_PACKED) -> dict:
    """The launch vitattn_fwd makes for these sizes on the current device
    (vitattn_fwd_shape): waves per workgroup, whether the waves split the
    keys of one query block, work items and workgroups."""
    vals = [ctypes.c_int() for _ in range(4)]
    rc = lib.vitattn_fwd_shape(int(B), int(H), int(N), int(D), int(layout),
                               *[ctypes.byref(x) for x in vals])
    if rc != OK:
        raise VitAttnError(rc, strerror(rc))
    waves, split, items, wgs = (x.value for x in vals)
    return {"waves": waves, "split_keys": bool(split), "items": items, "workgroups": wgs,
            "looping": wgs < items}


# vitattn_fwd itself, for the argument tuples fwd_args returns:
# fwd_c(*args) -> status, with no Python-level conversion.  The vectorcall
# module built beside the library converts the eleven arguments in a few
# hundred nanoseconds; the ctypes function (about 2 us) serves when that
# module has not been built.
try:
    from ._vitattn_ext import vitattn_fwd as fwd_c
except ImportError:
    fwd_c = lib.vitattn_fwd


def _layout_of(q_or_qkv, k, v, out):
    """Checks torch tensors as the C ABI expects them; returns
    (B, H, N, D, layout, out_shape), the layout carrying the fp16 flag for
    float16 tensors.  `out` may be None."""
    import torch

    if (k is None) != (v is None):
        raise ValueError("pass both k and v (separate layout) or neither (packed layout)")
    tensors = [q_or_qkv] + ([k, v] if k is not None else [])
    dtype = getattr(q_or_qkv, "dtype", None)
    if dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("inputs must be bfloat16 or float16 CUDA tensors")
    for t in tensors:
        if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
            raise TypeError("inputs must be CUDA tensors of one dtype, bfloat16 or float16")
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
    if dtype == torch.float16:
        layout |= DTYPE_FP16
    if out is not None:
        if (not isinstance(out, torch.Tensor) or out.dtype != dtype
                or tuple(out.shape) != out_shape or not out.is_contiguous()
                or out.device != q_or_qkv.device):
            raise ValueError(f"out must be a contiguous {dtype} tensor {out_shape} on the input device")
    return B, H, N, D, layout, out_shape


def fwd_args(q_or_qkv, k=None, v=None, *, out, scale: float | None = None, stream=None) -> tuple:
    """Checks a forward call once, as `fwd` does, and returns its C-ABI
    arguments (device addresses, sizes, scale, layout, stream handle) for
    repeated `fwd_raw(*args)` or `fwd_c(*args)` calls on the same tensors:
    loops that launch a fixed set of calls skip the per-call checks.  The tensors must stay
    alive, unmoved, while the arguments are used."""
    import torch

    if out is None:
        raise ValueError("fwd_args needs a preallocated out")
    B, H, N, D, layout, _ = _layout_of(q_or_qkv, k, v, out)
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if stream is None:
        stream = torch.cuda.current_stream(q_or_qkv.device)
    return (q_or_qkv.data_ptr(), k.data_ptr() if k is not None else None,
            v.data_ptr() if v is not None else None, out.data_ptr(), B, H, N, D, float(scale),
            layout, stream.cuda_stream)


def fwd(q_or_qkv, k=None, v=None, *, out=None, scale: float | None = None, stream=None):
    """O = softmax(scale * Q K^T) V per (image, head), on the GPU.

    Packed layout: `fwd(qkv)` with qkv a bf16 (or fp16) CUDA tensor
    [B, N, 3, H, D] (the fused qkv projection); returns out [B, N, H, D].
    Separate layout: `fwd(q, k, v)` with q, k, v CUDA tensors [B, H, N, D];
    returns out [B, H, N, D].  The output has the inputs' dtype.

    `scale` defaults to 1/sqrt(D).  `out` may be passed preallocated (same
    device and dtype, contiguous, output shape).  The kernel is enqueued on
    `stream` (a torch.cuda.Stream; default: the current stream) and the call
    returns without waiting.
    """
    import torch

    B, H, N, D, layout, out_shape = _layout_of(q_or_qkv, k, v, out)
    if out is None:
        out = torch.empty(out_shape, dtype=q_or_qkv.dtype, device=q_or_qkv.device)
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


def plan_create_raw(qkv_or_q, k, v, out, B: int, H: int, N: int, D: int, scale: float,
                    layout: int):
    """Direct call of vitattn_plan_create with lists of raw device addresses
    (k and v None for the packed layout).  Returns (status, handle)."""
    layers = len(qkv_or_q)
    arr = ctypes.c_void_p * max(layers, 1)

    def mk(xs):
        return None if xs is None else arr(*[x or None for x in xs])

    handle = ctypes.c_void_p()
    rc = lib.vitattn_plan_create(ctypes.byref(handle), layers, mk(qkv_or_q), mk(k), mk(v), mk(out),
                                 int(B), int(H), int(N), int(D), float(scale), int(layout))
    return rc, handle.value


def plan_launch_raw(handle, stream: int | None) -> int:
    return lib.vitattn_plan_launch(handle, stream or None)


def plan_destroy_raw(handle) -> int:
    return lib.vitattn_plan_destroy(handle)


class Plan:
    """A fixed sequence of forward calls recorded once into a HIP graph
    (vitattn_plan_create) and enqueued as one unit by `launch()`.

        plan = Plan([qkv_0, ..., qkv_L-1], outs=[out_0, ..., out_L-1])
        plan.launch()            # same results as fwd(qkv_l, out=out_l) for every l

    `inputs` holds one packed qkv tensor per call, or one (q, k, v) tuple per
    call for the separate layout; every call has the same shape.  `outs`
    defaults to new tensors (the `outs` attribute).  The tensors must stay
    alive, unmoved, while the plan is used: it holds references to them.
    """

    def __init__(self, inputs, outs=None, *, scale: float | None = None):
        import torch

        if not inputs:
            raise ValueError("a plan needs at least one call")
        calls = [(x, None, None) if isinstance(x, torch.Tensor) else tuple(x) for x in inputs]
        shape = None
        for (q, k, v) in calls:
            s = _layout_of(q, k, v, None)
            if shape is not None and s != shape:
                raise ValueError("every call of a plan must have the same shape and layout")
            shape = s
        B, H, N, D, layout, out_shape = shape
        if outs is None:
            outs = [torch.empty(out_shape, dtype=calls[0][0].dtype, device=calls[0][0].device)
                    for _ in calls]
        if len(outs) != len(calls):
            raise ValueError("one output per call")
        for (q, k, v), o in zip(calls, outs):
            _layout_of(q, k, v, o)
        if scale is None:
            scale = 1.0 / float(D) ** 0.5
        self.device = calls[0][0].device
        self.inputs, self.outs = calls, list(outs)
        sep = (layout & ~DTYPE_FP16) == LAYOUT_SEPARATE
        with torch.cuda.device(self.device):
            rc, self._handle = plan_create_raw(
                [c[0].data_ptr() for c in calls], [c[1].data_ptr() for c in calls] if sep else None,
                [c[2].data_ptr() for c in calls] if sep else None, [o.data_ptr() for o in self.outs],
                B, H, N, D, scale, layout)
        if rc != OK:
            self._handle = None
            raise VitAttnError(rc, strerror(rc))

    def launch(self, stream=None):
        """Enqueues every recorded call on `stream` (default: the current
        stream of the plan's device); returns without waiting."""
        import torch

        if self._handle is None:
            raise ValueError("the plan is closed")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        rc = plan_launch_raw(self._handle, stream.cuda_stream)
        if rc != OK:
            raise VitAttnError(rc, strerror(rc))
        return self.outs

    def close(self):
        if self._handle is not None:
            plan_destroy_raw(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def linear_raw(x: int, w: int, bias: int | None, residual: int | None, out: int, M: int, K: int,
               Nout: int, flags: int, stream: int | None) -> int:
    """Direct call of vitattn_linear with raw device addresses; returns the status."""
    return lib.vitattn_linear(x or None, w or None, bias or None, residual or None, out or None,
                              int(M), int(K), int(Nout), int(flags), stream or None)


def linear(x, w, bias=None, residual=None, *, out=None, stream=None):
    """out = x @ w.T + bias (+ residual) on the GPU (vitattn_linear).

    x: [..., K] CUDA tensor (bf16 or fp16, contiguous; the leading dimensions
    are the M tokens), w: [Nout, K] (the layer's weight as stored), bias:
    [Nout] or None, residual: None or a tensor of the output's shape (it may
    be `out` itself).  Returns out [..., Nout] in the inputs' dtype.  For the
    fused qkv projection of a ViT block, out [B, N, 3*H*D] viewed as
    [B, N, 3, H, D] is the packed input of `fwd`.
    """
    import torch

    dtype = getattr(x, "dtype", None)
    if dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("x must be a bfloat16 or float16 CUDA tensor")
    ts = [t for t in (x, w, bias, residual, out) if t is not None]
    for t in ts:
        if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
            raise TypeError("all tensors must be CUDA tensors of x's dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.device != x.device:
            raise ValueError("all tensors must be on the same device")
    if x.dim() < 1 or w.dim() != 2 or w.shape[1] != x.shape[-1]:
        raise ValueError(f"w must be [Nout, K] with K = x.shape[-1], got {tuple(w.shape)}")
    K = x.shape[-1]
    Nout = w.shape[0]
    M = x.numel() // K if K else 0
    out_shape = tuple(x.shape[:-1]) + (Nout,)
    if bias is not None and tuple(bias.shape) != (Nout,):
        raise ValueError(f"bias must be [{Nout}]")
    if residual is not None and tuple(residual.shape) != out_shape:
        raise ValueError(f"residual must be {out_shape}")
    if out is None:
        out = torch.empty(out_shape, dtype=dtype, device=x.device)
    elif tuple(out.shape) != out_shape:
        raise ValueError(f"out must be {out_shape}")
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    flags = DTYPE_FP16 if dtype == torch.float16 else 0
    rc = linear_raw(x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else None,
                    residual.data_ptr() if residual is not None else None, out.data_ptr(), M, K,
                    Nout, flags, stream.cuda_stream)
    if rc != OK:
        raise VitAttnError(rc, strerror(rc))
    return out
