"""Facts the definition of softmax attention fixes, checked on the HIP path
through the C ABI (the GPU side of the oracle's pins):

  * the hand-computed 4-token case (tests/golden/four_token_case.json: the
    closed forms evaluated with Python's decimal module, no oracle involved);
  * affinity in V: O(Q, K, 2V) = 2 O(Q, K, V) bit for bit (scaling by 2 is
    exact in every step), and O(Q, K, V + b) = O(Q, K, V) + b within the bar;
  * key-shift invariance: adding one vector u to every key adds q_i . u to
    every logit of row i, which the softmax removes;
  * invariance under a joint permutation of the keys and values;
  * layout equivalence: the same logical values in the packed and in the
    separate layout give the same output bits.

The method these pins hold the kernel to is exact softmax attention (the Pi0
Flash Attention tutorial, section 1 and the section 4.2 table: the fast
kernel leaves the outputs unchanged).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from gpu_util import LAYOUT_PACKED, LAYOUT_SEPARATE, assert_parity, bits_of, logical, to_device
from workloads import LayerInputs, f32_to_bf16_bits, f32_to_f16_bits

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "four_token_case.json")


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def va():
    import vit_self_attention_amd
    return vit_self_attention_amd


def _run(va, li, layout, scale, device, fmt="bf16"):
    import torch
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    ts = [None if a is None else
          torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).to(device)
          for a in li.in_layout(layout)]
    o = va.fwd(ts[0], ts[1], ts[2], scale=scale)
    torch.cuda.synchronize(device)
    return o


def _bits_logical(o, layout):
    b = bits_of(o)
    return b.transpose(0, 2, 1, 3) if layout == LAYOUT_SEPARATE else b


# ---------------------------------------------------------------- G5: the 4-token case

@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("layout", [LAYOUT_PACKED, LAYOUT_SEPARATE])
@pytest.mark.parametrize("D", [64, 72])
def test_four_token_closed_form(dev, va, D, layout, fmt):
    """Every (image, head) of a 2 x 3 batch holds the golden case; all
    inputs are exact in bf16 and fp16.  Column 0 must match the closed form
    within the 16-bit rounding of the weights and of the output, column 1
    (V = 1 for every key) is exactly 1, and the other columns exactly 0."""
    with open(GOLDEN) as f:
        case = json.load(f)
    N, B, H = case["N"], 2, 3
    rnd = f32_to_f16_bits if fmt == "f16" else f32_to_bf16_bits
    q = np.zeros((B, N, H, D), np.float32)
    k = np.zeros((B, N, H, D), np.float32)
    v = np.zeros((B, N, H, D), np.float32)
    q[..., 0] = np.asarray(case["q_col0"], np.float32)[None, :, None]
    k[..., 0] = np.asarray(case["k_col0"], np.float32)[None, :, None]
    v[..., 0] = np.asarray(case["v_col0"], np.float32)[None, :, None]
    v[..., 1] = np.asarray(case["v_col1"], np.float32)[None, :, None]
    li = LayerInputs(rnd(q), rnd(k), rnd(v))
    o = _run(va, li, layout, case["scale"], dev, fmt)
    got = logical(o, layout)
    want0 = np.asarray(case["expected_o_col0"])[None, :, None]
    # weights rounded to 8 (bf16) or 11 (fp16) significant bits move O by at
    # most 2^-8 (2^-11) of max|V - O| <= 3; the output's rounding adds half
    # an ulp of a value below 4
    bits = 11 if fmt == "f16" else 8
    bound = 3.0 * 2.0 ** -bits + 2.0 ** (2 - bits)
    err = np.abs(got[..., 0] - want0)
    print(f"4-token D={D} layout={layout} {fmt}: col0 max err {err.max():.3e} (bound {bound:.3e})",
          flush=True)
    assert err.max() <= bound
    assert np.all(got[..., 1] == 1.0)
    assert np.all(got[..., 2:] == 0.0)


# ---------------------------------------------------------------- P8: invariants

def _grid_values(rng, shape, lo, hi, step):
    """Values on a grid of `step`, exact in bf16 (at most 8 significant bits)."""
    n = int(round((hi - lo) / step))
    return (lo + step * rng.integers(0, n + 1, size=shape)).astype(np.float32)


@pytest.mark.parametrize("D", [64, 72])
def test_affine_in_v(dev, va, D):
    rng = np.random.default_rng(200 + D)
    B, N, H = 3, 277, 4
    q = f32_to_bf16_bits(rng.standard_normal((B, N, H, D)).astype(np.float32) * np.float32(2.0))
    k = f32_to_bf16_bits(rng.standard_normal((B, N, H, D)).astype(np.float32) * np.float32(2.0))
    # |V + b| <= 4 on a grid of 1/32 (exact in bf16), so every output lies
    # below 4 in magnitude and rounds with an error of at most 2^-7
    vf = _grid_values(rng, (B, N, H, D), -2.0, 2.0, 1.0 / 32)
    bvec = _grid_values(rng, (1, 1, H, D), -2.0, 2.0, 0.25)
    scale = 1.0 / math.sqrt(D)
    base = _run(va, LayerInputs(q, k, f32_to_bf16_bits(vf)), LAYOUT_PACKED, scale, dev)
    twice = _run(va, LayerInputs(q, k, f32_to_bf16_bits(2.0 * vf)), LAYOUT_PACKED, scale, dev)
    # scaling every value by 2 is exact in the inputs, the fp32 products and
    # sums, and the output's rounding: the result doubles bit for bit
    assert np.array_equal(logical(twice, LAYOUT_PACKED), 2.0 * logical(base, LAYOUT_PACKED))
    shifted = _run(va, LayerInputs(q, k, f32_to_bf16_bits(vf + bvec)), LAYOUT_PACKED, scale, dev)
    assert_parity(logical(shifted, LAYOUT_PACKED), logical(base, LAYOUT_PACKED) + bvec,
                  f"O(V + b) vs O(V) + b, D={D}")


@pytest.mark.parametrize("D", [64, 72])
def test_key_shift_invariance(dev, va, D):
    """K_l <- K_l + u for every key l: row i's logits all move by
    scale * q_i . u (tens of logit units here), P is unchanged."""
    rng = np.random.default_rng(210 + D)
    B, N, H = 2, 333, 3
    q = _grid_values(rng, (B, N, H, D), -4.0, 4.0, 0.0625)
    k = _grid_values(rng, (B, N, H, D), -4.0, 4.0, 0.0625)
    u = _grid_values(rng, (B, 1, H, D), -3.0, 3.0, 0.0625)  # k + u stays on the grid: exact
    v = f32_to_bf16_bits(_grid_values(rng, (B, N, H, D), -2.0, 2.0, 1.0 / 64))
    scale = 1.0 / math.sqrt(D)
    shift = np.abs(np.einsum("bnhd,bohd->bnh", q.astype(np.float64), u.astype(np.float64))).max()
    assert shift * scale > 10.0  # the shift is large
    base = _run(va, LayerInputs(f32_to_bf16_bits(q), f32_to_bf16_bits(k), v), LAYOUT_PACKED, scale, dev)
    moved = _run(va, LayerInputs(f32_to_bf16_bits(q), f32_to_bf16_bits(k + u), v), LAYOUT_PACKED,
                 scale, dev)
    # |O| <= 2: each output is within 2^-8 (its rounding) plus the weights'
    # rounding of the exact value, so the two runs agree within the bar
    assert_parity(logical(moved, LAYOUT_PACKED), logical(base, LAYOUT_PACKED),
                  f"key shift, D={D}")
    ref = oracle.attention(*LayerInputs(f32_to_bf16_bits(q), f32_to_bf16_bits(k + u), v).in_layout(
        LAYOUT_PACKED), LAYOUT_PACKED, B, H, N, D, scale)
    assert_parity(logical(moved, LAYOUT_PACKED), ref, f"shifted keys vs oracle, D={D}")


@pytest.mark.parametrize("D", [64, 72])
def test_joint_key_value_permutation(dev, va, D):
    rng = np.random.default_rng(220 + D)
    B, N, H = 2, 401, 3
    q, k = (f32_to_bf16_bits(rng.standard_normal((B, N, H, D)).astype(np.float32) * np.float32(2.5))
            for _ in range(2))
    v = f32_to_bf16_bits(_grid_values(rng, (B, N, H, D), -2.0, 2.0, 1.0 / 64))
    perm = rng.permutation(N)
    scale = 1.0 / math.sqrt(D)
    base = _run(va, LayerInputs(q, k, v), LAYOUT_PACKED, scale, dev)
    perm_out = _run(va, LayerInputs(q, np.ascontiguousarray(k[:, perm]), np.ascontiguousarray(v[:, perm])),
                    LAYOUT_PACKED, scale, dev)
    assert_parity(logical(perm_out, LAYOUT_PACKED), logical(base, LAYOUT_PACKED),
                  f"joint K/V permutation, D={D}")
    ref = oracle.attention(*LayerInputs(q, k, v).in_layout(LAYOUT_PACKED), LAYOUT_PACKED, B, H, N, D,
                           scale)
    assert_parity(logical(perm_out, LAYOUT_PACKED), ref, f"permuted vs oracle, D={D}")


# ---------------------------------------------------------------- P9: layouts

@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("B,H,N,D", [(2, 16, 256, 72), (1, 12, 197, 64), (24, 16, 257, 64),
                                     (6, 16, 729, 72), (3, 5, 1, 72)])
def test_layouts_give_identical_bits(dev, va, B, H, N, D, fmt):
    """The kernel's arithmetic does not depend on the strides, so the packed
    [B,N,3,H,D] and the separate [B,H,N,D] layouts of the same values give
    the same output bits (in [B,N,H,D] and [B,H,N,D] order respectively)."""
    rng = np.random.default_rng(230 + N)
    rnd = f32_to_f16_bits if fmt == "f16" else f32_to_bf16_bits
    li = LayerInputs(*(rnd(rng.standard_normal((B, N, H, D)).astype(np.float32) * np.float32(2.0))
                       for _ in range(3)))
    scale = 1.0 / math.sqrt(D)
    packed = _bits_logical(_run(va, li, LAYOUT_PACKED, scale, dev, fmt), LAYOUT_PACKED)
    separate = _bits_logical(_run(va, li, LAYOUT_SEPARATE, scale, dev, fmt), LAYOUT_SEPARATE)
    assert np.array_equal(packed, separate)
