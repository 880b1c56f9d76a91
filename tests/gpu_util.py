"""Helpers shared by the GPU tests: moving seeded bf16 bits to the device,
calling the library through its C ABI, and comparing with the oracle."""
from __future__ import annotations

import numpy as np

from workloads import LAYOUT_PACKED, LAYOUT_SEPARATE, LayerInputs

MAX_ABS = 2e-2   # tolerance for bf16 inputs, max over all elements
MEAN_ABS = 2e-3  # and mean over all elements


def to_device(bits, device):
    import torch
    if bits is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def run_gpu(li: LayerInputs, layout: int, scale: float, device, out=None):
    """Runs vitattn on one layer's inputs; returns float64 [B, N, H, D]."""
    import torch
    import vit_self_attention_amd as va

    arrs = li.in_layout(layout)
    ts = [to_device(a, device) for a in arrs]
    o = va.fwd(ts[0], ts[1], ts[2], scale=scale, out=out)
    torch.cuda.synchronize(device)
    return logical(o, layout)


def logical(o, layout):
    """Device output -> float64 numpy in logical order [B, N, H, D]."""
    got = o.float().cpu().numpy().astype(np.float64)
    if layout == LAYOUT_SEPARATE:
        got = got.transpose(0, 2, 1, 3)
    return got


def bits_of(o):
    """Device bf16 tensor -> uint16 bit patterns (numpy)."""
    import torch
    return o.view(torch.int16).cpu().numpy().view(np.uint16)


def errors(got, ref):
    err = np.abs(got - ref)
    return float(err.max()), float(err.mean())


def assert_parity(got, ref, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = errors(got, ref)
    print(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e}"


__all__ = ["MAX_ABS", "MEAN_ABS", "to_device", "run_gpu", "logical", "bits_of", "errors",
           "assert_parity", "LAYOUT_PACKED", "LAYOUT_SEPARATE"]
