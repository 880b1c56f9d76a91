"""Parity of the HIP path with the fp64 oracle, element by element, through
the C ABI.  Tolerance for bf16 inputs: max-abs <= 2e-2 and mean-abs <= 2e-3.
"""
import math

import numpy as np
import pytest

import oracle
from gpu_util import (LAYOUT_PACKED, LAYOUT_SEPARATE, assert_parity, bits_of, logical, run_gpu,
                      to_device)
from workloads import WORKLOADS, LayerInputs, Workload, f32_to_bf16_bits, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def va():
    import vit_self_attention_amd
    return vit_self_attention_amd


def _oracle(li, layout, scale):
    B, N, H, D = li.q.shape
    return oracle.attention(*li.in_layout(layout), layout, B, H, N, D, scale)


# ---------------------------------------------------------------- full workloads

@pytest.mark.parametrize("key", sorted(WORKLOADS))
def test_workload_parity_all_layers(dev, va, key):
    """Every layer of every workload at its full size, in the launch
    configuration the benchmark times, against the oracle on all elements."""
    wl = WORKLOADS[key]
    print(f"[parity] {key}: {wl.name}", flush=True)
    worst = 0.0
    for layer in range(wl.layers):
        li = make_layer(wl, layer)
        got = run_gpu(li, wl.layout, wl.scale, dev)
        ref = _oracle(li, wl.layout, wl.scale)
        assert_parity(got, ref, f"{key} layer {layer}")
        worst = max(worst, float(np.abs(got - ref).max()))
    print(f"[parity] {key}: worst max_abs over {wl.layers} layers = {worst:.3e}", flush=True)


# ---------------------------------------------------------------- ragged sizes

# includes last key tiles of 1, 32 and 33 keys after an odd and an even
# number of full tiles (288 = 4*64 + 32, 321 = 5*64 + 1, 353 = 5*64 + 33)
RAGGED_N = [1, 2, 3, 31, 32, 33, 63, 64, 65, 101, 127, 128, 129, 197, 255, 256, 257, 288, 300,
            321, 353]


@pytest.mark.parametrize("D", [64, 72])
@pytest.mark.parametrize("layout", [LAYOUT_PACKED, LAYOUT_SEPARATE])
@pytest.mark.parametrize("N", RAGGED_N)
def test_ragged_parity(dev, va, N, layout, D):
    """Sizes spanning several tiles with ragged query and key tails."""
    wl = Workload("t", "ragged", B=2, N=N, H=3, D=D, layout=layout, layers=1, kind="iid",
                  index=40 + D)
    li = make_layer(wl, N)
    got = run_gpu(li, layout, wl.scale, dev)
    assert_parity(got, _oracle(li, layout, wl.scale), f"N={N} D={D} layout={layout}")


@pytest.mark.parametrize("D", [64, 72])
@pytest.mark.parametrize("N", [65, 200, 729])
def test_stress_logits_parity(dev, va, N, D):
    """Logit std ~8 with 10% near-one-hot rows: the running max must be exact."""
    wl = Workload("t", "stress", B=2, N=N, H=4, D=D, layout=LAYOUT_PACKED, layers=1,
                  kind="stress", index=50 + D)
    li = make_layer(wl, 0)
    got = run_gpu(li, LAYOUT_PACKED, wl.scale, dev)
    assert_parity(got, _oracle(li, LAYOUT_PACKED, wl.scale), f"stress N={N} D={D}")


@pytest.mark.parametrize("B,H,N", [(1, 1, 729), (4, 16, 729), (96, 16, 64), (1, 48, 129),
                                   (8, 16, 256), (12, 16, 200), (6, 16, 729)])
def test_grid_shapes(dev, va, B, H, N):
    """Grids with every wave count the launcher picks, and uneven XCD splits.
    (8, 16, 256) and (12, 16, 200) are short sequences on 256 and 384
    four-wave workgroups; (6, 16, 729), one GPU's share of
    48 images at 384 px over 8 GPUs, gives 576 items on the 512 looping
    workgroups that fit on the chip at once, 64 of them taking a second."""
    wl = Workload("t", "grid", B=B, N=N, H=H, D=72, layout=LAYOUT_PACKED, layers=1, kind="iid",
                  index=60)
    li = make_layer(wl, B * 1000 + N)
    got = run_gpu(li, LAYOUT_PACKED, wl.scale, dev)
    assert_parity(got, _oracle(li, LAYOUT_PACKED, wl.scale), f"grid B={B} H={H} N={N}")


@pytest.mark.parametrize("D", [64, 72])
def test_long_sequence_looping_workgroups(dev, va, D):
    """N = 2048 with enough (image, head, query block) items for the
    looping-workgroup kernel (B*H*16 = 1024 items), full comparison: long
    tile streams, many items per workgroup, lazy rescales across 32 tiles."""
    wl = Workload("t", "long", B=4, N=2048, H=16, D=D, layout=LAYOUT_PACKED, layers=1,
                  kind="stress", index=70 + D)
    li = make_layer(wl, 0)
    got = run_gpu(li, LAYOUT_PACKED, wl.scale, dev)
    assert_parity(got, _oracle(li, LAYOUT_PACKED, wl.scale), f"long N=2048 D={D}")


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("N,D", [(131071, 72), (100001, 64)])
def test_very_long_sequence_sampled_rows(dev, va, N, D, fmt):
    """One image, two heads, about 10^5 tokens: 1.5-2k key tiles per item
    (streams far longer than any encoder's), ragged last key tiles of 63
    and 33 keys and last query blocks of 127 and 33 rows, stress logits
    (std ~8) with boosted rows; checked on sampled rows against the
    oracle's row entry point."""
    import torch
    wl = Workload("t", "very long", B=1, N=N, H=2, D=D, layout=LAYOUT_PACKED, layers=1,
                  kind="stress", index=80 + D)
    assert va.fwd_shape(1, 2, N, D)["looping"]
    li = make_layer(wl, 0, fmt=fmt)
    arrs = li.in_layout(LAYOUT_PACKED)
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    qkv = torch.from_numpy(np.ascontiguousarray(arrs[0]).view(np.int16)).view(dt).to(dev)
    print(f"[very long] N={N} D={D} {fmt}", flush=True)
    o = va.fwd(qkv, scale=wl.scale)
    torch.cuda.synchronize(dev)
    got = logical(o, LAYOUT_PACKED)
    rng = np.random.default_rng(81 + D)
    R = 96
    rows = np.stack([np.zeros(R, np.int64), rng.integers(0, 2, R), rng.integers(0, N, R)], 1)
    rows[:6, 2] = [0, 1, 63, 64, N - 2, N - 1]
    ref = oracle.attention_rows(*arrs, LAYOUT_PACKED, 1, 2, N, D, wl.scale, rows, fmt=fmt)
    got_rows = np.stack([got[b, i, h] for b, h, i in rows])
    assert np.all(np.isfinite(got_rows))
    err = np.abs(got_rows - ref)
    tmax, tmean = (1e-2, 1e-3) if fmt == "f16" else (2e-2, 2e-3)
    print(f"[very long] N={N} D={D} {fmt}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= tmax and err.mean() <= tmean


def test_separate_layout_full_size_sampled_rows(dev, va):
    """The 384 px workload's shape and values in the separate [B,H,N,D]
    layout, run by the looping-workgroup kernel, checked on 256 sampled
    (image, head, query) rows, including the ragged last query block."""
    wl = WORKLOADS["c5"]
    li = make_layer(wl, 0)
    B, N, H, D = li.q.shape
    arrs = li.in_layout(LAYOUT_SEPARATE)
    got = run_gpu(li, LAYOUT_SEPARATE, wl.scale, dev)
    rng = np.random.default_rng(71)
    rows = np.stack([rng.integers(0, B, 256), rng.integers(0, H, 256), rng.integers(0, N, 256)], 1)
    rows[:8, 2] = [0, 1, 127, 128, 639, 640, 727, 728]
    ref = oracle.attention_rows(*arrs, LAYOUT_SEPARATE, B, H, N, D, wl.scale, rows)
    got_rows = np.stack([got[b, i, h] for b, h, i in rows])
    err = np.abs(got_rows - ref)
    print(f"separate c5 sampled: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


# ---------------------------------------------------------------- special cases

def _rand(rng, shape, std=1.0):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


@pytest.mark.parametrize("D", [64, 72])
def test_single_token_returns_v_bitwise(dev, va, D):
    """N = 1: p = 1 and l = 1, so O = V exactly."""
    rng = np.random.default_rng(1)
    li = LayerInputs(_rand(rng, (5, 1, 7, D)), _rand(rng, (5, 1, 7, D)), _rand(rng, (5, 1, 7, D)))
    for layout in (LAYOUT_PACKED, LAYOUT_SEPARATE):
        import torch
        arrs = li.in_layout(layout)
        ts = [to_device(a, dev) for a in arrs]
        o = va.fwd(ts[0], ts[1], ts[2], scale=0.125)
        torch.cuda.synchronize(dev)
        got = bits_of(o)
        if layout == LAYOUT_SEPARATE:
            got = got.transpose(0, 2, 1, 3)
        assert np.array_equal(got, li.v)


@pytest.mark.parametrize("D", [64, 72])
def test_identical_keys_and_zero_scale_give_mean(dev, va, D):
    rng = np.random.default_rng(2)
    B, N, H = 2, 150, 3
    q = _rand(rng, (B, N, H, D), 3.0)
    v = _rand(rng, (B, N, H, D))
    k = np.ascontiguousarray(np.broadcast_to(_rand(rng, (B, 1, H, D)), (B, N, H, D)))
    vf = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mean = np.broadcast_to(vf.mean(axis=1, keepdims=True), (B, N, H, D))
    got = run_gpu(LayerInputs(q, k, v), LAYOUT_PACKED, 1 / math.sqrt(D), dev)
    assert_parity(got, mean, "identical keys")
    got = run_gpu(LayerInputs(q, _rand(rng, (B, N, H, D)), v), LAYOUT_PACKED, 0.0, dev)
    assert_parity(got, mean, "scale 0")


@pytest.mark.parametrize("D", [64, 72])
def test_negative_scale(dev, va, D):
    rng = np.random.default_rng(3)
    B, N, H = 2, 97, 2
    li = LayerInputs(_rand(rng, (B, N, H, D)), _rand(rng, (B, N, H, D)), _rand(rng, (B, N, H, D)))
    got = run_gpu(li, LAYOUT_SEPARATE, -0.2, dev)
    assert_parity(got, _oracle(li, LAYOUT_SEPARATE, -0.2), "negative scale")


@pytest.mark.parametrize("D", [64, 72])
def test_constant_value_channel_is_one(dev, va, D):
    """A value channel equal to 1 for every key comes out as 1 (rows of P sum
    to 1) within bf16 rounding."""
    rng = np.random.default_rng(4)
    B, N, H = 2, 257, 3
    v = _rand(rng, (B, N, H, D))
    v[..., 5] = f32_to_bf16_bits(np.ones((B, N, H), np.float32))
    li = LayerInputs(_rand(rng, (B, N, H, D), 2.8), _rand(rng, (B, N, H, D), 2.8), v)
    got = run_gpu(li, LAYOUT_PACKED, 1 / math.sqrt(D), dev)
    assert np.max(np.abs(got[..., 5] - 1.0)) <= 2.0 ** -8


@pytest.mark.parametrize("D", [64, 72])
def test_dominant_key_one_hot(dev, va, D):
    """Q_i = K_t with a large scale: key t leads every other key of row i by
    tens of logit units, so O_i = V_t up to bf16 rounding."""
    rng = np.random.default_rng(5)
    B, N, H = 1, 190, 2
    k = _rand(rng, (B, N, H, D))
    target = rng.integers(0, N, size=(N, H))
    q = np.empty_like(k)
    for h in range(H):
        q[0, :, h, :] = k[0, target[:, h], h, :]
    kf = (k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    v = _rand(rng, (B, N, H, D))
    scale = 4.0
    for h in range(H):
        s = scale * kf[0, target[:, h], h, :] @ kf[0, :, h, :].T
        top2 = np.sort(s, axis=1)[:, -2:]
        assert np.all(top2[:, 1] - top2[:, 0] > 20.0)   # the case is what it claims
    got = run_gpu(LayerInputs(q, k, v), LAYOUT_PACKED, scale, dev)
    vf = (v.astype(np.uint32) << 16).view(np.float32)
    for h in range(H):
        expect = vf[0, target[:, h], h, :]
        assert np.max(np.abs(got[0, :, h, :] - expect)) <= np.abs(expect).max() * 2.0 ** -8


def test_query_permutation_is_bitwise(dev, va):
    """Each query row's arithmetic does not depend on its position."""
    import torch
    rng = np.random.default_rng(6)
    B, N, H, D = 2, 229, 3, 72
    q, k, v = (_rand(rng, (B, N, H, D)) for _ in range(3))
    perm = rng.permutation(N)
    outs = []
    for qq in (q, np.ascontiguousarray(q[:, perm])):
        arrs = LayerInputs(qq, k, v).in_layout(LAYOUT_SEPARATE)
        ts = [to_device(a, dev) for a in arrs]
        o = va.fwd(ts[0], ts[1], ts[2], scale=0.1)
        torch.cuda.synchronize(dev)
        outs.append(bits_of(o))
    assert np.array_equal(outs[1], outs[0][:, :, perm])


def test_deterministic(dev, va):
    import torch
    wl = WORKLOADS["c5"]
    li = make_layer(wl, 0, B=4)
    qkv = to_device(li.packed(), dev)
    o1 = va.fwd(qkv, scale=wl.scale)
    o2 = va.fwd(qkv, scale=wl.scale)
    torch.cuda.synchronize(dev)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_prepared_call_matches_fwd(dev, va):
    """fwd_args + fwd_raw (checked once, called many times) gives fwd's bits,
    in both layouts."""
    import torch
    wl = WORKLOADS["c3"]
    li = make_layer(wl, 5)
    qkv = to_device(li.packed(), dev)
    ref = va.fwd(qkv, scale=wl.scale)
    out = torch.empty_like(ref)
    args = va.fwd_args(qkv, out=out, scale=wl.scale)
    for _ in range(3):
        assert va.fwd_raw(*args) == va.OK
        assert va.fwd_c(*args) == va.OK
    torch.cuda.synchronize(dev)
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))
    q, k, v = (to_device(a, dev) for a in li.in_layout(LAYOUT_SEPARATE))
    ref = va.fwd(q, k, v, scale=wl.scale)
    out = torch.empty_like(ref)
    assert va.fwd_raw(*va.fwd_args(q, k, v, out=out, scale=wl.scale)) == va.OK
    torch.cuda.synchronize(dev)
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))
    with pytest.raises(ValueError):
        va.fwd_args(qkv, out=None)


@pytest.mark.parametrize("N", [1, 33, 101, 257])
def test_no_writes_outside_out(dev, va, N):
    """Guard regions before and after `out` keep their pattern (ragged tails
    never store past the last token)."""
    import torch
    B, H, D = 3, 5, 72
    rng = np.random.default_rng(7)
    li = LayerInputs(*(_rand(rng, (B, N, H, D)) for _ in range(3)))
    qkv = to_device(li.packed(), dev)
    n_out = B * N * H * D
    guard = 4096  # elements, a multiple of 8 so `out` stays 16-byte aligned
    buf = torch.full((guard + n_out + guard,), -12345.0, dtype=torch.bfloat16, device=dev)
    out = buf[guard:guard + n_out].view(B, N, H, D)
    va.fwd(qkv, out=out, scale=0.12)
    torch.cuda.synchronize(dev)
    pattern = torch.tensor(-12345.0, dtype=torch.bfloat16)
    assert torch.all(buf[:guard].cpu() == pattern)
    assert torch.all(buf[guard + n_out:].cpu() == pattern)
    assert_parity(logical(out, LAYOUT_PACKED), _oracle(li, LAYOUT_PACKED, 0.12), f"guarded N={N}")


def test_empty_problem_leaves_out_untouched(dev, va):
    import torch
    qkv = torch.zeros(2, 0, 3, 4, 64, dtype=torch.bfloat16, device=dev)
    out = va.fwd(qkv)
    torch.cuda.synchronize(dev)
    assert out.shape == (2, 0, 4, 64)


def test_errors_raise(dev, va):
    import torch
    qkv = torch.zeros(1, 8, 3, 2, 80, dtype=torch.bfloat16, device=dev)
    with pytest.raises(va.VitAttnError) as e:
        va.fwd(qkv)
    assert e.value.status == va._binding.ERR_UNSUPPORTED_D
    qkv = torch.zeros(1, 8, 3, 2, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(va.VitAttnError) as e:
        va.fwd(qkv, scale=float("nan"))
    assert e.value.status == va._binding.ERR_BAD_SCALE


@pytest.mark.parametrize("D", [64, 72])
def test_large_values_with_growing_row_maxima(dev, va, D):
    """bf16 values near 2^66 (about 7e19) with row maxima that grow by some
    40 (log2 units) per key tile, so the accumulator is rescaled tile after
    tile: the weights stay below 2^32 before each rescale, the fp32 sums of
    weight times value stay finite (with weights up to 2^64 they would
    overflow), and the result scaled back by 2^-66 meets the bar."""
    rng = np.random.default_rng(91)
    B, N, H = 1, 600, 2
    scale = 1 / math.sqrt(D)
    q = rng.standard_normal((B, N, H, D)).astype(np.float32) * np.float32(0.5)
    k = rng.standard_normal((B, N, H, D)).astype(np.float32) * np.float32(0.5)
    # logit of key j grows by 40 / log2(e) per 64 keys along channel 0
    step = 40.0 / 1.4426950408889634 / 64.0
    q[..., 0] = 8.0
    k[..., 0] = (np.arange(N, dtype=np.float32) * np.float32(step / (8.0 * scale)))[None, :, None]
    v = rng.standard_normal((B, N, H, D)).astype(np.float32)
    big = np.float32(2.0 ** 66)
    li = LayerInputs(f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v * big))
    got = run_gpu(li, LAYOUT_PACKED, scale, dev)
    assert np.all(np.isfinite(got)), "non-finite output for large values"
    ref = _oracle(li, LAYOUT_PACKED, scale)
    assert_parity(got / 2.0 ** 66, ref / 2.0 ** 66, "values near 2^66, growing maxima")
