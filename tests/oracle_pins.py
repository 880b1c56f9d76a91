"""Pins for the fp64 oracle: checks against facts that the definition of
softmax attention fixes, independent of the oracle's own code.

Each pin is a function `pin_*(lib)` taking a loaded oracle library (ctypes)
and raising AssertionError when the oracle disagrees with the fact.  The
tests run them on the real oracle (all must pass) and on deliberately broken
copies of it (each copy must fail at least one), which shows that a
plausible slip in the oracle -- a dropped term, a wrong sign or index, a
transposed operand -- cannot go unnoticed.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from workloads import (LAYOUT_PACKED, LAYOUT_SEPARATE, LayerInputs, bf16_bits_to_f32,
                       f16_bits_to_f32, f32_to_bf16_bits, f32_to_f16_bits)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(x):
    """float array that is exact in bf16 -> uint16 bits (asserts exactness)."""
    x = np.asarray(x, dtype=np.float32)
    b = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(b), x), "test input not exact in bf16"
    return b


def _rand_bits(rng, shape, std=1.0):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


def _run(lib, q, k, v, scale, layout=LAYOUT_PACKED, want_probs=False, fmt="bf16"):
    """q, k, v: uint16 [B, N, H, D].  Returns the oracle's O (and P)."""
    B, N, H, D = q.shape
    li = LayerInputs(q, k, v)
    a, kk, vv = li.in_layout(layout)
    return oracle.attention(a, kk, vv, layout, B, H, N, D, scale, want_probs=want_probs, lib=lib,
                            fmt=fmt)


def _bits16(x):
    """float array that is exact in fp16 -> uint16 bits (asserts exactness)."""
    x = np.asarray(x, dtype=np.float32)
    b = f32_to_f16_bits(x)
    assert np.array_equal(f16_bits_to_f32(b), x), "test input not exact in fp16"
    return b


def _f(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------- pins

def pin_four_token_closed_form(lib):
    """Worked 4-token case: outputs are closed forms in e (tests/golden)."""
    with open(os.path.join(GOLDEN, "four_token_case.json")) as f:
        case = json.load(f)
    # the fixture's digits agree with the closed forms evaluated here
    for i in range(4):
        z = sum(math.exp(i * l) for l in range(4))
        o0 = sum(l * math.exp(i * l) for l in range(4)) / z
        assert abs(o0 - case["expected_o_col0"][i]) < 1e-13
    for D in (64, 72):
        for layout in (LAYOUT_PACKED, LAYOUT_SEPARATE):
            q = np.zeros((1, 4, 1, D), np.float32)
            k = np.zeros_like(q)
            v = np.zeros_like(q)
            q[0, :, 0, 0] = case["q_col0"]
            k[0, :, 0, 0] = case["k_col0"]
            v[0, :, 0, 0] = case["v_col0"]
            v[0, :, 0, 1] = case["v_col1"]
            o, p = _run(lib, _bits(q), _bits(k), _bits(v), case["scale"], layout, want_probs=True)
            np.testing.assert_allclose(o[0, :, 0, 0], case["expected_o_col0"], rtol=0, atol=1e-12)
            np.testing.assert_allclose(o[0, :, 0, 1], case["expected_o_col1"], rtol=0, atol=1e-12)
            assert np.all(o[0, :, 0, 2:] == 0.0)
            np.testing.assert_allclose(p[0, 0], np.array(case["expected_p"]), rtol=0, atol=1e-12)


def pin_rows_sum_to_one(lib):
    """Every row of P is a probability vector."""
    rng = np.random.default_rng(11)
    for (B, N, H, D, std) in [(2, 37, 3, 64, 1.0), (1, 50, 2, 72, 2.8)]:
        q = _rand_bits(rng, (B, N, H, D), std)
        k = _rand_bits(rng, (B, N, H, D), std)
        v = _rand_bits(rng, (B, N, H, D))
        _, p = _run(lib, q, k, v, 1 / math.sqrt(D), want_probs=True)
        assert np.all(p >= 0.0)
        assert np.max(np.abs(p.sum(axis=-1) - 1.0)) <= 1e-12


def pin_identical_keys_give_mean(lib):
    """All keys equal: every query attends uniformly, O_i = mean_j V_j.
    The same holds for scale = 0 with arbitrary keys."""
    rng = np.random.default_rng(12)
    B, N, H, D = 2, 29, 3, 72
    q = _rand_bits(rng, (B, N, H, D), 3.0)
    v = _rand_bits(rng, (B, N, H, D))
    k1 = _rand_bits(rng, (B, 1, H, D))
    k = np.ascontiguousarray(np.broadcast_to(k1, (B, N, H, D)))
    mean_v = _f(v).mean(axis=1, keepdims=True)
    o = _run(lib, q, k, v, 1 / math.sqrt(D))
    np.testing.assert_allclose(o, np.broadcast_to(mean_v, o.shape), rtol=0, atol=1e-12)
    k = _rand_bits(rng, (B, N, H, D))
    o = _run(lib, q, k, v, 0.0)
    np.testing.assert_allclose(o, np.broadcast_to(mean_v, o.shape), rtol=0, atol=1e-12)


def pin_query_permutation_equivariance(lib):
    """Permuting the queries permutes the output rows the same way."""
    rng = np.random.default_rng(13)
    B, N, H, D = 1, 31, 2, 64
    q = _rand_bits(rng, (B, N, H, D))
    k = _rand_bits(rng, (B, N, H, D))
    v = _rand_bits(rng, (B, N, H, D))
    perm = rng.permutation(N)
    o = _run(lib, q, k, v, 0.125)
    for layout in (LAYOUT_PACKED, LAYOUT_SEPARATE):
        o_p = _run(lib, np.ascontiguousarray(q[:, perm]), k, v, 0.125, layout)
        assert np.array_equal(o_p, o[:, perm])


def pin_key_value_permutation_invariance(lib):
    """Permuting keys and values together leaves the output unchanged."""
    rng = np.random.default_rng(14)
    B, N, H, D = 2, 23, 2, 72
    q = _rand_bits(rng, (B, N, H, D))
    k = _rand_bits(rng, (B, N, H, D))
    v = _rand_bits(rng, (B, N, H, D))
    perm = rng.permutation(N)
    o = _run(lib, q, k, v, 0.2, LAYOUT_SEPARATE)
    o2 = _run(lib, q, np.ascontiguousarray(k[:, perm]), np.ascontiguousarray(v[:, perm]), 0.2,
              LAYOUT_SEPARATE)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)


def pin_dominant_key_one_hot(lib):
    """A key whose logit exceeds every other by >= 40 takes all the weight:
    O_i = V_j to within e^-40.  Logits up to ~1e3 also check that the
    softmax stays finite (no overflow)."""
    rng = np.random.default_rng(15)
    B, N, H, D = 1, 20, 2, 64
    q = np.zeros((B, N, H, D), np.float32)
    k = np.zeros((B, N, H, D), np.float32)
    target = rng.integers(0, N, size=(N, H))
    for h in range(H):
        for j in range(N):
            k[0, j, h, j % D] = 4.0          # K_j = 4 e_{j mod D}
        for i in range(N):
            q[0, i, h, target[i, h] % D] = 64.0   # Q_i . K_t = 256, others 0
    v = _rand_bits(rng, (B, N, H, D))
    for scale in (1.0, 4.0):               # gaps 256 and 1024 in the logits
        o = _run(lib, _bits(q), _bits(k), v, scale)
        assert np.all(np.isfinite(o))
        for h in range(H):
            expect = _f(v)[0, target[:, h], h, :]
            np.testing.assert_allclose(o[0, :, h, :], expect, rtol=0, atol=1e-12)


def pin_two_keys_logistic(lib):
    """N = 2: O_i = V_1 + sigmoid(s_i0 - s_i1) (V_0 - V_1), a closed form."""
    rng = np.random.default_rng(16)
    B, N, H, D = 1, 2, 2, 72
    q = _rand_bits(rng, (B, N, H, D))
    k = _rand_bits(rng, (B, N, H, D))
    v = _rand_bits(rng, (B, N, H, D))
    scale = 0.3
    o = _run(lib, q, k, v, scale)
    qf, kf, vf = _f(q), _f(k), _f(v)
    for h in range(H):
        for i in range(N):
            s0 = scale * float(np.dot(qf[0, i, h], kf[0, 0, h]))
            s1 = scale * float(np.dot(qf[0, i, h], kf[0, 1, h]))
            w = 1.0 / (1.0 + math.exp(-(s0 - s1)))
            expect = vf[0, 1, h] + w * (vf[0, 0, h] - vf[0, 1, h])
            np.testing.assert_allclose(o[0, i, h], expect, rtol=0, atol=1e-12)


def pin_single_token_is_identity(lib):
    """N = 1: P = [1], so O = V exactly."""
    rng = np.random.default_rng(17)
    for D in (64, 72):
        B, N, H = 3, 1, 4
        q = _rand_bits(rng, (B, N, H, D))
        k = _rand_bits(rng, (B, N, H, D))
        v = _rand_bits(rng, (B, N, H, D))
        for layout in (LAYOUT_PACKED, LAYOUT_SEPARATE):
            o = _run(lib, q, k, v, 0.125, layout)
            assert np.array_equal(o, _f(v))


def pin_affine_in_values(lib):
    """O(Q, K, a V + c) = a O(Q, K, V) + c (rows of P sum to 1)."""
    rng = np.random.default_rng(18)
    B, N, H, D = 1, 17, 2, 64
    q = _rand_bits(rng, (B, N, H, D))
    k = _rand_bits(rng, (B, N, H, D))
    vg = rng.integers(-8, 9, size=(B, N, H, D)).astype(np.float32) / 4   # exact grid
    a, c = 2.0, 0.5
    o1 = _run(lib, q, k, _bits(vg), 0.125)
    o2 = _run(lib, q, k, _bits(a * vg + c), 0.125)
    np.testing.assert_allclose(o2, a * o1 + c, rtol=0, atol=1e-12)


def pin_key_shift_invariance(lib):
    """Adding one vector u to every key shifts row i's logits by a constant,
    which the softmax removes: O is unchanged."""
    rng = np.random.default_rng(19)
    B, N, H, D = 1, 19, 2, 72
    q = _rand_bits(rng, (B, N, H, D))
    kg = rng.integers(-8, 9, size=(B, N, H, D)).astype(np.float32) / 4
    u = rng.integers(-8, 9, size=(B, 1, H, D)).astype(np.float32) / 4
    v = _rand_bits(rng, (B, N, H, D))
    o1 = _run(lib, q, _bits(kg), v, 0.1)
    o2 = _run(lib, q, _bits(kg + u), v, 0.1)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)


def pin_negative_scale(lib):
    """scale * (Q.K) = (-scale) * ((-Q).K): negating Q and the scale leaves O unchanged."""
    rng = np.random.default_rng(20)
    B, N, H, D = 1, 13, 2, 64
    q = _rand_bits(rng, (B, N, H, D))
    k = _rand_bits(rng, (B, N, H, D))
    v = _rand_bits(rng, (B, N, H, D))
    o1 = _run(lib, q, k, v, 0.125)
    o2 = _run(lib, q ^ np.uint16(0x8000), k, v, -0.125)
    assert np.array_equal(o1, o2)


def pin_layout_invariance(lib):
    """The same logical values give the same output in both input layouts."""
    rng = np.random.default_rng(21)
    B, N, H, D = 2, 21, 3, 72
    q = _rand_bits(rng, (B, N, H, D))
    k = _rand_bits(rng, (B, N, H, D))
    v = _rand_bits(rng, (B, N, H, D))
    o_p = _run(lib, q, k, v, 0.11, LAYOUT_PACKED)
    o_s = _run(lib, q, k, v, 0.11, LAYOUT_SEPARATE)
    assert np.array_equal(o_p, o_s)


def pin_library_sdpa(lib):
    """Agreement with torch's scaled_dot_product_attention evaluated in
    float64 on the CPU (an independent library routine for the same
    definition), over several images and heads, with ragged N."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(22)
    for (B, N, H, D, std) in [(2, 1, 3, 64, 1.0), (2, 5, 3, 72, 1.0), (3, 33, 4, 64, 1.0),
                              (2, 47, 2, 72, 2.8)]:
        q = _rand_bits(rng, (B, N, H, D), std)
        k = _rand_bits(rng, (B, N, H, D), std)
        v = _rand_bits(rng, (B, N, H, D))
        scale = 1 / math.sqrt(D)
        o = _run(lib, q, k, v, scale)
        tq, tk, tv = (torch.from_numpy(_f(t).transpose(0, 2, 1, 3).copy()) for t in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy().transpose(0, 2, 1, 3)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def pin_brute_force_tiny(lib):
    """Tiny cases against a direct evaluation with Python floats and math.exp."""
    rng = np.random.default_rng(23)
    for (N, D) in [(1, 1), (2, 2), (3, 1), (4, 2), (5, 3), (8, 2)]:
        B, H = 1, 2
        q = _rand_bits(rng, (B, N, H, D))
        k = _rand_bits(rng, (B, N, H, D))
        v = _rand_bits(rng, (B, N, H, D))
        o = _run(lib, q, k, v, 0.7)
        qf, kf, vf = _f(q), _f(k), _f(v)
        for h in range(H):
            for i in range(N):
                w = [math.exp(0.7 * math.fsum(qf[0, i, h, d] * kf[0, j, h, d] for d in range(D)))
                     for j in range(N)]
                z = math.fsum(w)
                for d in range(D):
                    ref = math.fsum(w[j] * vf[0, j, h, d] for j in range(N)) / z
                    assert abs(o[0, i, h, d] - ref) <= 1e-12, (N, D, h, i, d)


def pin_rows_entry_matches_closed_forms(lib):
    """The row-sampling entry point: 4-token closed form, N = 1 identity and
    identical-keys mean, on selected (b, h, i) rows."""
    with open(os.path.join(GOLDEN, "four_token_case.json")) as f:
        case = json.load(f)
    D = 72
    q = np.zeros((1, 4, 1, D), np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    q[0, :, 0, 0] = case["q_col0"]
    k[0, :, 0, 0] = case["k_col0"]
    v[0, :, 0, 0] = case["v_col0"]
    v[0, :, 0, 1] = case["v_col1"]
    packed = LayerInputs(_bits(q), _bits(k), _bits(v)).packed()
    rows = [(0, 0, 3), (0, 0, 1)]
    o = oracle.attention_rows(packed, None, None, LAYOUT_PACKED, 1, 1, 4, D, 0.125, rows, lib=lib)
    np.testing.assert_allclose(o[:, 0], [case["expected_o_col0"][3], case["expected_o_col0"][1]],
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[:, 1], 1.0, rtol=0, atol=1e-12)
    rng = np.random.default_rng(24)
    B, N, H = 2, 9, 3
    qb = _rand_bits(rng, (B, N, H, D))
    vb = _rand_bits(rng, (B, N, H, D))
    kb = np.ascontiguousarray(np.broadcast_to(_rand_bits(rng, (B, 1, H, D)), (B, N, H, D)))
    a, kk, vv = LayerInputs(qb, kb, vb).in_layout(LAYOUT_SEPARATE)
    rows = [(1, 2, 0), (0, 1, 8), (1, 0, 4)]
    o = oracle.attention_rows(a, kk, vv, LAYOUT_SEPARATE, B, H, N, D, 0.5, rows, lib=lib)
    mean_v = _f(vb).mean(axis=1)
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(o[r], mean_v[b, h], rtol=0, atol=1e-12)


# ------------------------------------------------------------- fp16 inputs

def pin_widening_of_every_pattern(lib):
    """Every one of the 65536 patterns widens to the value numpy's own
    float16 (IEEE binary16) and bfloat16-as-top-half-of-float32 conversions
    give (NaN patterns to NaN)."""
    bits = np.arange(65536, dtype=np.uint16)
    # widening the signalling-NaN patterns raises numpy's "invalid value" flag
    with np.errstate(invalid="ignore"):
        refs = (("f16", bits.view(np.float16).astype(np.float64)),
                ("bf16", (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)))
    for fmt, ref in refs:
        got = np.array([oracle.widen(int(b), fmt, lib=lib) for b in bits])
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), fmt
        assert np.array_equal(got[~nan], ref[~nan]), fmt


def pin_four_token_closed_form_fp16(lib):
    """The worked 4-token case with fp16 inputs (all its values are exact in
    fp16) gives the same closed-form outputs."""
    with open(os.path.join(GOLDEN, "four_token_case.json")) as f:
        case = json.load(f)
    for layout in (LAYOUT_PACKED, LAYOUT_SEPARATE):
        q = np.zeros((1, 4, 1, 72), np.float32)
        k = np.zeros_like(q)
        v = np.zeros_like(q)
        q[0, :, 0, 0] = case["q_col0"]
        k[0, :, 0, 0] = case["k_col0"]
        v[0, :, 0, 0] = case["v_col0"]
        v[0, :, 0, 1] = case["v_col1"]
        o = _run(lib, _bits16(q), _bits16(k), _bits16(v), case["scale"], layout, fmt="f16")
        np.testing.assert_allclose(o[0, :, 0, 0], case["expected_o_col0"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(o[0, :, 0, 1], case["expected_o_col1"], rtol=0, atol=1e-12)
        assert np.all(o[0, :, 0, 2:] == 0.0)


def pin_formats_agree_on_shared_values(lib):
    """Values exact in both bf16 and fp16 (8 significant bits, exponents
    inside fp16's normal range) give bitwise the same output in either
    format: only the decoding of the bits differs."""
    rng = np.random.default_rng(31)
    B, N, H, D = 2, 19, 3, 72
    for layout in (LAYOUT_PACKED, LAYOUT_SEPARATE):
        t = [np.ldexp(rng.integers(-255, 256, (B, N, H, D)).astype(np.float32), -6)
             for _ in range(3)]
        ob = _run(lib, *(_bits(x) for x in t), 0.09, layout, fmt="bf16")
        oh = _run(lib, *(_bits16(x) for x in t), 0.09, layout, fmt="f16")
        assert np.array_equal(ob, oh)


def pin_library_sdpa_fp16(lib):
    """fp16 inputs against torch's scaled_dot_product_attention in float64
    on the CPU, with values only fp16 represents (11 significant bits)."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(32)
    for (B, N, H, D, std) in [(2, 7, 3, 64, 1.0), (2, 41, 2, 72, 2.8)]:
        t = [f32_to_f16_bits(rng.standard_normal((B, N, H, D)).astype(np.float32) * np.float32(s))
             for s in (std, std, 1.0)]
        scale = 1 / math.sqrt(D)
        o = _run(lib, *t, scale, fmt="f16")
        tq, tk, tv = (torch.from_numpy(f16_bits_to_f32(x).astype(np.float64).transpose(0, 2, 1, 3).copy())
                      for x in t)
        ref = F.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy().transpose(0, 2, 1, 3)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


ALL_PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}
