"""Parity of the fp16 variant (VITATTN_DTYPE_FP16) with the fp64 oracle on
the same fp16 inputs, through the C ABI.

Tolerance, from the arithmetic: fp16 keeps 11 significant bits against
bf16's 8, so the output's final rounding costs at most 2^-11 relative
(about 0.004 absolute at |O| < 8), and the weights rounded to fp16 for the
P V product add at most 2^-11 of max|V - O| (about 0.005 at |V| < 5); the
fp32 accumulation is far below both.  Bound used: max-abs <= 1e-2 and
mean-abs <= 1e-3 over all elements, half of the bf16 bar.
"""
import math

import numpy as np
import pytest

import oracle
from gpu_util import LAYOUT_PACKED, LAYOUT_SEPARATE, bits_of, logical
from workloads import WORKLOADS, LayerInputs, Workload, f16_bits_to_f32, f32_to_f16_bits, make_layer

pytestmark = pytest.mark.gpu

MAX_ABS_F16 = 1e-2
MEAN_ABS_F16 = 1e-3


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def va():
    import vit_self_attention_amd
    return vit_self_attention_amd


def _to_dev16(bits, device):
    import torch
    if bits is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(device)


def _run16(va, li, layout, scale, device):
    import torch
    ts = [_to_dev16(a, device) for a in li.in_layout(layout)]
    o = va.fwd(ts[0], ts[1], ts[2], scale=scale)
    torch.cuda.synchronize(device)
    assert o.dtype == torch.float16
    return logical(o, layout), o


def _oracle16(li, layout, scale):
    B, N, H, D = li.q.shape
    return oracle.attention(*li.in_layout(layout), layout, B, H, N, D, scale, fmt="f16")


def _check(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    print(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= MAX_ABS_F16 and err.mean() <= MEAN_ABS_F16, what


@pytest.mark.parametrize("key", sorted(WORKLOADS))
def test_fp16_workload_parity_all_layers(dev, va, key):
    """Every layer of every workload, its float32 draws rounded to fp16."""
    wl = WORKLOADS[key]
    print(f"[parity fp16] {key}: {wl.name}", flush=True)
    for layer in range(wl.layers):
        li = make_layer(wl, layer, fmt="f16")
        got, _ = _run16(va, li, wl.layout, wl.scale, dev)
        _check(got, _oracle16(li, wl.layout, wl.scale), f"fp16 {key} layer {layer}")


@pytest.mark.parametrize("D", [64, 72])
@pytest.mark.parametrize("layout", [LAYOUT_PACKED, LAYOUT_SEPARATE])
@pytest.mark.parametrize("N", [1, 2, 33, 64, 65, 129, 257, 300])
def test_fp16_ragged_parity(dev, va, N, layout, D):
    wl = Workload("t", "ragged fp16", B=2, N=N, H=3, D=D, layout=layout, layers=1, kind="iid",
                  index=70 + D)
    li = make_layer(wl, N, fmt="f16")
    got, _ = _run16(va, li, layout, wl.scale, dev)
    _check(got, _oracle16(li, layout, wl.scale), f"fp16 N={N} D={D} layout={layout}")


@pytest.mark.parametrize("D", [64, 72])
def test_fp16_growing_logits_rescale(dev, va, D):
    """Row maxima that grow tile after tile by far more than 2^8 (the fp16
    kernel's lazy bound), so the accumulator is rescaled again and again:
    key j carries a component proportional to j along each query."""
    rng = np.random.default_rng(80 + D)
    B, N, H = 1, 700, 2
    q = rng.standard_normal((B, N, H, D)).astype(np.float32)
    k = rng.standard_normal((B, N, H, D)).astype(np.float32) * np.float32(0.3)
    # logit of key j grows by 8 * 64 * j / N * scale, about 87 in log2 units
    # over the row (some 8 per 64-key tile)
    q[..., 0] = 8.0
    k[..., 0] = np.linspace(0.0, 64.0, N, dtype=np.float32)[None, :, None]
    v = rng.standard_normal((B, N, H, D)).astype(np.float32)
    li = LayerInputs(f32_to_f16_bits(q), f32_to_f16_bits(k), f32_to_f16_bits(v))
    scale = 1 / math.sqrt(D)
    got, _ = _run16(va, li, LAYOUT_PACKED, scale, dev)
    _check(got, _oracle16(li, LAYOUT_PACKED, scale), f"fp16 growing logits D={D}")


@pytest.mark.parametrize("D", [64, 72])
def test_fp16_single_token_is_exact(dev, va, D):
    """N = 1: the weight is exactly 1 and O = V bit for bit."""
    rng = np.random.default_rng(90)
    t = [f32_to_f16_bits(rng.standard_normal((3, 1, 5, D)).astype(np.float32)) for _ in range(3)]
    li = LayerInputs(*t)
    _, o = _run16(va, li, LAYOUT_PACKED, 0.3, dev)
    assert np.array_equal(bits_of(o), li.v)


def test_fp16_plan_replays_bitwise(dev, va):
    import torch
    wl = WORKLOADS["c3"]
    calls, eager = [], []
    for layer in range(4):
        li = make_layer(wl, layer, fmt="f16")
        t = _to_dev16(li.packed(), dev)
        calls.append(t)
        eager.append(bits_of(va.fwd(t, scale=wl.scale)))
    plan = va.Plan(calls, scale=wl.scale)
    try:
        for _ in range(2):
            for o in plan.outs:
                o.zero_()
            plan.launch()
            torch.cuda.synchronize(dev)
            for o, want in zip(plan.outs, eager):
                assert o.dtype == torch.float16
                assert np.array_equal(bits_of(o), want)
    finally:
        plan.close()


def test_mixed_dtypes_rejected(dev, va):
    import torch
    q = torch.zeros((1, 2, 8, 64), dtype=torch.float16, device=dev)
    k = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(TypeError):
        va.fwd(q, k, k)
    with pytest.raises(ValueError):
        va.fwd(q, q, q, out=torch.empty((1, 2, 8, 64), dtype=torch.bfloat16, device=dev))
