"""Parity of vitattn_linear (the qkv and output projections around the
attention) with the fp64 oracle, through the C ABI.

Tolerance, from the arithmetic: the products of 16-bit inputs are exact in
fp32 and are summed in fp32, which over K <= 4096 terms stays within
2^-12 * S, S = sum_k |x_k w_k| + |bias| + |residual| (the worst case is
K * 2^-24 * S); the output is then rounded once, by at most half an ulp:
2^-8 of |out| for bf16 (8 significant bits), 2^-11 for fp16 (11 bits).
Bar per element: |got - ref| <= 2^-8 |ref| (bf16) or 2^-10 |ref| (fp16),
plus 2^-12 * S.
"""
import numpy as np
import pytest

from oracle import linear as lo
from workloads import f32_to_bf16_bits, f32_to_f16_bits

pytestmark = pytest.mark.gpu

ROUND = {"bf16": f32_to_bf16_bits, "f16": f32_to_f16_bits}
REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -10}


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def va():
    import vit_self_attention_amd
    return vit_self_attention_amd


def _dev(bits, fmt, device):
    import torch
    if bits is None:
        return None
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).to(device)


def _host(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _inputs(seed, M, K, Nout, fmt, bias=True, residual=False, wstd=None):
    rng = np.random.default_rng(seed)
    wstd = wstd if wstd is not None else 1.0 / np.sqrt(K)  # an initialised layer's scale
    x = ROUND[fmt](rng.standard_normal((M, K)).astype(np.float32))
    w = ROUND[fmt](rng.standard_normal((Nout, K)).astype(np.float32) * np.float32(wstd))
    b = ROUND[fmt](rng.standard_normal(Nout).astype(np.float32) * np.float32(0.1)) if bias else None
    r = ROUND[fmt](rng.standard_normal((M, Nout)).astype(np.float32)) if residual else None
    return x, w, b, r


def _check(got_bits, x, w, b, r, fmt, rows=None, what=""):
    ref = lo.linear(x, w, b, r, fmt) if rows is None else lo.linear_rows(x, w, b, r, rows, fmt)
    xs = np.abs(lo.widen(x if rows is None else np.asarray(x)[rows], fmt))
    S = xs @ np.abs(lo.widen(w, fmt)).T
    if b is not None:
        S = S + np.abs(lo.widen(b, fmt))[None, :]
    if r is not None:
        S = S + np.abs(lo.widen(r if rows is None else np.asarray(r)[rows], fmt))
    got = lo.widen(got_bits, fmt)
    err = np.abs(got - ref)
    bound = REL[fmt] * np.abs(ref) + 2.0 ** -12 * S
    worst = float((err / bound).max())
    print(f"{what}: max_abs={err.max():.3e} worst err/bound={worst:.3f}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert worst <= 1.0, what


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_qkv_projection_siglip224(dev, va, fmt):
    """The fused qkv projection of SigLIP-So400m at 224 px, two views
    (M = 2*256 tokens, 1152 -> 3*16*72), every element; its output viewed
    as [B, N, 3, H, D] is accepted by the attention."""
    import torch
    M, K, Nout = 512, 1152, 3456
    x, w, b, _ = _inputs(1, M, K, Nout, fmt)
    out = va.linear(_dev(x, fmt, dev), _dev(w, fmt, dev), _dev(b, fmt, dev))
    torch.cuda.synchronize(dev)
    _check(_host(out), x, w, b, None, fmt, what=f"qkv 224 {fmt}")
    o = va.fwd(out.view(2, 256, 3, 16, 72))
    torch.cuda.synchronize(dev)
    assert o.shape == (2, 256, 16, 72) and bool(torch.isfinite(o.float()).all())


def test_qkv_projection_siglip384_sampled_rows(dev, va):
    """SigLIP at 384 px, 48 images (M = 34992, the 256 x 256 tile kernel),
    checked on sampled rows including the ragged last tile."""
    import torch
    M, K, Nout = 48 * 729, 1152, 3456
    x, w, b, _ = _inputs(2, M, K, Nout, "bf16")
    out = _host(va.linear(_dev(x, "bf16", dev), _dev(w, "bf16", dev), _dev(b, "bf16", dev)))
    torch.cuda.synchronize(dev)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 257, M - 1],
                                     rng.integers(0, M, 58)]))
    _check(out[rows], x, w, b, None, "bf16", rows=rows, what="qkv 384 sampled")


@pytest.mark.parametrize("fmt,K,Nout,resid", [("f16", 1152, 3456, False), ("bf16", 64, 2048, True)])
def test_streaming_store_path(dev, va, fmt, K, Nout, resid):
    """Outputs above 128 MiB go out with non-temporal stores (a separate
    kernel instantiation of the 256 x 256 tile shape): the fp16 qkv
    projection at 384 px x 48, and a bf16 call with a residual (M = 34992,
    Nout = 2048: 143 MB), on sampled rows."""
    import torch
    M = 48 * 729
    assert M * Nout * 2 > 128 << 20
    x, w, b, r = _inputs(40 + K, M, K, Nout, fmt, residual=resid)
    out = va.linear(*[_dev(t, fmt, dev) for t in (x, w, b)], _dev(r, fmt, dev))
    torch.cuda.synchronize(dev)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.integers(0, M, 40)]))
    _check(_host(out)[rows], x, w, b, r, fmt, rows=rows, what=f"streaming {fmt} K={K} Nout={Nout}")


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_output_projection_with_residual(dev, va, fmt):
    """out = o w^T + b + x, with a separate output and in place (out is x)."""
    import torch
    M, K, Nout = 512, 1152, 1152
    o, w, b, r = _inputs(3, M, K, Nout, fmt, residual=True)
    td = [_dev(t, fmt, dev) for t in (o, w, b, r)]
    y = va.linear(td[0], td[1], td[2], residual=td[3])
    torch.cuda.synchronize(dev)
    _check(_host(y), o, w, b, r, fmt, what=f"proj {fmt}")
    inplace = td[3].clone()
    va.linear(td[0], td[1], td[2], residual=inplace, out=inplace)
    torch.cuda.synchronize(dev)
    assert np.array_equal(_host(inplace), _host(y))


@pytest.mark.parametrize("M", [1, 7, 127, 129, 300])
@pytest.mark.parametrize("K,Nout", [(32, 8), (64, 136), (96, 264), (1152, 72)])
def test_ragged_shapes(dev, va, M, K, Nout):
    import torch
    x, w, b, r = _inputs(10 + M + K, M, K, Nout, "bf16", residual=(M % 2 == 1))
    td = [_dev(t, "bf16", dev) for t in (x, w, b, r)]
    y = va.linear(td[0], td[1], td[2], residual=td[3])
    torch.cuda.synchronize(dev)
    _check(_host(y), x, w, b, r, "bf16", what=f"M={M} K={K} Nout={Nout}")


# one shape per tile configuration the launcher picks, each with ragged M and
# Nout: 256 x 256, 128 x 128, 64 x 128 and 64 x 64 tiles
@pytest.mark.parametrize("M,K,Nout", [(4100, 64, 4104), (2100, 96, 2056), (1000, 64, 2056),
                                      (300, 96, 264)])
def test_every_tile_config(dev, va, M, K, Nout):
    import torch
    x, w, b, r = _inputs(30 + M, M, K, Nout, "bf16", residual=True)
    td = [_dev(t, "bf16", dev) for t in (x, w, b, r)]
    y = va.linear(td[0], td[1], td[2], residual=td[3])
    torch.cuda.synchronize(dev)
    _check(_host(y), x, w, b, r, "bf16", what=f"M={M} K={K} Nout={Nout}")


def test_no_bias_no_residual_and_determinism(dev, va):
    import torch
    M, K, Nout = 1000, 256, 512
    x, w, _, _ = _inputs(20, M, K, Nout, "bf16", bias=False)
    xd, wd = _dev(x, "bf16", dev), _dev(w, "bf16", dev)
    y1 = _host(va.linear(xd, wd))
    y2 = _host(va.linear(xd, wd))
    torch.cuda.synchronize(dev)
    assert np.array_equal(y1, y2)
    _check(y1, x, w, None, None, "bf16", what="no bias")


def test_binding_rejects_bad_shapes(dev, va):
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        va.linear(x, torch.zeros((8, 32), dtype=torch.bfloat16, device=dev))
    with pytest.raises(TypeError):
        va.linear(x, torch.zeros((8, 64), dtype=torch.float16, device=dev))
    with pytest.raises(va.VitAttnError):
        va.linear(torch.zeros((4, 48), dtype=torch.bfloat16, device=dev),
                  torch.zeros((8, 48), dtype=torch.bfloat16, device=dev))


def test_attention_sublayer_composition(dev, va):
    """The attention sublayer of a SigLIP block on the library's kernels:
    qkv = x Wqkv^T + b (vitattn_linear), viewed as the packed [B,N,3,H,D]
    input of vitattn_fwd, whose [B,N,H,D] output viewed as [B,N,H*D] feeds
    the output projection with bias and the residual x.  Each stage is
    checked against the oracle on exactly the bits the GPU stage consumed."""
    import math
    import torch
    import oracle
    B, N, H, D = 2, 256, 16, 72
    E = H * D
    rng = np.random.default_rng(40)
    x = ROUND["bf16"](rng.standard_normal((B * N, E)).astype(np.float32))
    wqkv = ROUND["bf16"](rng.standard_normal((3 * E, E)).astype(np.float32) * np.float32(1 / math.sqrt(E)))
    bqkv = ROUND["bf16"](rng.standard_normal(3 * E).astype(np.float32) * np.float32(0.1))
    wo = ROUND["bf16"](rng.standard_normal((E, E)).astype(np.float32) * np.float32(1 / math.sqrt(E)))
    bo = ROUND["bf16"](rng.standard_normal(E).astype(np.float32) * np.float32(0.1))
    xd = _dev(x, "bf16", dev)
    qkv = va.linear(xd, _dev(wqkv, "bf16", dev), _dev(bqkv, "bf16", dev))
    o = va.fwd(qkv.view(B, N, 3, H, D), scale=1 / math.sqrt(D))
    y = va.linear(o.view(B * N, E), _dev(wo, "bf16", dev), _dev(bo, "bf16", dev), residual=xd)
    torch.cuda.synchronize(dev)
    qkv_bits, o_bits, y_bits = _host(qkv), _host(o), _host(y)
    _check(qkv_bits, x, wqkv, bqkv, None, "bf16", what="sublayer qkv")
    ref_o = oracle.attention(qkv_bits.reshape(B, N, 3, H, D), None, None, 1, B, H, N, D, 1 / math.sqrt(D))
    err = np.abs(lo.widen(o_bits).reshape(B, N, H, D) - ref_o)
    print(f"sublayer attention: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    _check(y_bits, o_bits.reshape(B * N, E), wo, bo, x, "bf16", what="sublayer proj + residual")
