"""Pins for the fp64 linear-layer oracle (oracle/linear.py), on the CPU:
facts the definition out = x w^T + bias + residual fixes, checked without
the oracle's own code path."""
import math

import numpy as np
import pytest

from oracle import linear as lo
from workloads import f32_to_bf16_bits, f32_to_f16_bits

ROUND = {"bf16": f32_to_bf16_bits, "f16": f32_to_f16_bits}


def _rand(rng, shape, fmt, std=1.0):
    return ROUND[fmt](rng.standard_normal(shape).astype(np.float32) * np.float32(std))


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_brute_force_tiny(fmt):
    """Python floats and math.fsum over every (m, n)."""
    rng = np.random.default_rng(1)
    M, K, Nout = 3, 5, 4
    x, w, b, r = (_rand(rng, s, fmt) for s in ((M, K), (Nout, K), (Nout,), (M, Nout)))
    got = lo.linear(x, w, b, r, fmt)
    xf, wf, bf, rf = (lo.widen(t, fmt) for t in (x, w, b, r))
    for m in range(M):
        for n in range(Nout):
            ref = math.fsum([xf[m, k] * wf[n, k] for k in range(K)] + [bf[n], rf[m, n]])
            assert abs(got[m, n] - ref) <= 1e-12 * (1 + abs(ref)), (m, n)


def test_widen_matches_numpy_formats():
    bits = np.arange(65536, dtype=np.uint16)
    f16 = lo.widen(bits, "f16")
    ref16 = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(f16), np.isnan(ref16))
    assert np.array_equal(f16[~np.isnan(f16)], ref16[~np.isnan(ref16)])
    bf = lo.widen(np.array([0x3f80, 0xc000, 0x0001, 0x7f7f], np.uint16), "bf16")
    assert bf[0] == 1.0 and bf[1] == -2.0 and bf[2] == 2.0 ** -133
    assert bf[3] == (2 - 2 ** -7) * 2.0 ** 127


def test_identity_and_permutation_weights():
    """w = I gives x + bias + residual exactly; a permutation weight permutes
    the input features."""
    rng = np.random.default_rng(2)
    M, K = 6, 32
    x = _rand(rng, (M, K), "bf16")
    eye = ROUND["bf16"](np.eye(K, dtype=np.float32))
    b = _rand(rng, (K,), "bf16")
    r = _rand(rng, (M, K), "bf16")
    got = lo.linear(x, eye, b, r)
    assert np.array_equal(got, lo.widen(x) + lo.widen(b)[None, :] + lo.widen(r))
    perm = rng.permutation(K)
    pw = ROUND["bf16"](np.eye(K, dtype=np.float32)[perm])
    assert np.array_equal(lo.linear(x, pw), lo.widen(x)[:, perm])


def test_rows_entry_matches_full():
    rng = np.random.default_rng(3)
    M, K, Nout = 40, 64, 24
    x, w, b, r = (_rand(rng, s, "f16") for s in ((M, K), (Nout, K), (Nout,), (M, Nout)))
    rows = [0, 17, 39, 5]
    assert np.array_equal(lo.linear_rows(x, w, b, r, rows, "f16"), lo.linear(x, w, b, r, "f16")[rows])


def test_linearity_in_x():
    """out(x1 + x2) - bias = out(x1) - bias + out(x2) - bias for inputs whose
    sum is exact in bf16 (small integers)."""
    rng = np.random.default_rng(4)
    M, K, Nout = 5, 32, 16
    x1 = rng.integers(-8, 9, (M, K)).astype(np.float32)
    x2 = rng.integers(-8, 9, (M, K)).astype(np.float32)
    w = _rand(rng, (Nout, K), "bf16")
    b = _rand(rng, (Nout,), "bf16")
    o1 = lo.linear(ROUND["bf16"](x1), w, b)
    o2 = lo.linear(ROUND["bf16"](x2), w, b)
    o12 = lo.linear(ROUND["bf16"](x1 + x2), w, b)
    np.testing.assert_allclose(o12 - lo.widen(b), (o1 - lo.widen(b)) + (o2 - lo.widen(b)),
                               rtol=0, atol=1e-9)
