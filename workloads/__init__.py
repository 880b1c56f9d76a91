"""Seeded synthetic inputs for the vision-encoder self-attention forward.

This module only draws and lays out input bits. It holds none of the
attention arithmetic, so the oracle and the HIP path can both be fed from it
without sharing any step of the method.

Workloads (shapes follow the pages' vision encoders):
  * ViT-B/16 at 224 px gives 196 patches + CLS = 197 tokens; at 160 px,
    100 patches + CLS = 101 tokens (the resolution sweep in "Pi0 VLA model
    inference performance analysis", section 3.2).
  * ViT-L/14 at 224 px gives 256 patches + CLS = 257 tokens (same page,
    section 3.1, names ViT-L/14 as the encoder).
  * SigLIP-So400m/14 (the pi0 vision tower, "Realtime-VLA V2", section 1.1.2)
    at 224 px gives 16x16 = 256 tokens and at 384 px 27x27 = 729 tokens
    (384 px is the input size in the VLA speed-up article, section 2.1).
  * Camera views become the batch: three views in the Pi0 Flash Attention
    tutorial (section 4.2), two views in Realtime-VLA (section 1.1.1).

Every random number comes from numpy's PCG64 with a seed fixed by the
workload and the layer, so the inputs are reproducible bit for bit.
Values are drawn in float32, transformed in float32, and rounded to bfloat16
with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

LAYOUT_SEPARATE = 0  # q, k, v each [B, H, N, D]; out [B, H, N, D]
LAYOUT_PACKED = 1    # one buffer [B, N, 3, H, D]; out [B, N, H, D]


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload."""

    key: str            # short id, c1 .. c5
    name: str           # human-readable name with its sizes
    B: int
    N: int
    H: int
    D: int
    layout: int
    layers: int         # number of independent layer calls timed back to back
    kind: str           # value recipe, see make_layer()
    index: int          # 1-based workload number, enters the seeds
    scale: float = field(default=0.0)

    def __post_init__(self):
        if self.scale == 0.0:
            object.__setattr__(self, "scale", 1.0 / math.sqrt(self.D))

    @property
    def flops_per_layer(self) -> int:
        """Algorithmic flops of one layer call: Q K^T plus P V, 2 flops per MAC."""
        return 4 * self.B * self.H * self.N * self.N * self.D

    @property
    def bytes_per_layer(self) -> int:
        """Algorithmic HBM bytes: read Q, K, V once and write O once, bf16."""
        return 2 * 4 * self.B * self.N * self.H * self.D

    def seed(self, layer: int) -> int:
        return 1000 * self.index + layer

    @property
    def aux_seed(self) -> int:
        return 1000 * self.index + 999


WORKLOADS = {
    "c1": Workload("c1", "ViT-B/16 224px, 1 image, separate Q/K/V (B=1,N=197,H=12,D=64)",
                   B=1, N=197, H=12, D=64, layout=LAYOUT_SEPARATE, layers=1,
                   kind="iid", index=1),
    "c2": Workload("c2", "ViT-B/16 160px, 3 views, packed QKV (B=3,N=101,H=12,D=64), 12 layers",
                   B=3, N=101, H=12, D=64, layout=LAYOUT_PACKED, layers=12,
                   kind="iid", index=2),
    "c3": Workload("c3", "SigLIP-So400m/14 224px, 2 views, packed QKV (B=2,N=256,H=16,D=72), 27 layers",
                   B=2, N=256, H=16, D=72, layout=LAYOUT_PACKED, layers=27,
                   kind="gamma", index=3),
    "c4": Workload("c4", "ViT-L/14 224px, 3 views x batch 8, packed QKV (B=24,N=257,H=16,D=64), 24 layers",
                   B=24, N=257, H=16, D=64, layout=LAYOUT_PACKED, layers=24,
                   kind="iid", index=4),
    "c5": Workload("c5", "SigLIP-So400m/14 384px, 3 views x batch 16, packed QKV (B=48,N=729,H=16,D=72), "
                   "logit std ~8 with 10% near-one-hot rows",
                   B=48, N=729, H=16, D=72, layout=LAYOUT_PACKED, layers=1,
                   kind="stress", index=5),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE fp16 (numpy's conversion: round to
    nearest, ties to even).  Returns the 16-bit patterns as uint16; inputs
    must lie inside fp16's range."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size and float(np.abs(x).max()) >= 65520.0:
        raise ValueError("value outside the fp16 range")
    return x.astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of fp16 bit patterns to float32."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


ROUND = {"bf16": f32_to_bf16_bits, "f16": f32_to_f16_bits}
WIDEN = {"bf16": bf16_bits_to_f32, "f16": f16_bits_to_f32}


@dataclass
class LayerInputs:
    """Bits of one layer's Q, K, V in the logical order [B, N, H, D]."""

    q: np.ndarray  # uint16 [B, N, H, D]
    k: np.ndarray
    v: np.ndarray

    def packed(self) -> np.ndarray:
        """The fused-QKV activation [B, N, 3, H, D] (uint16)."""
        return np.ascontiguousarray(np.stack([self.q, self.k, self.v], axis=2))

    def separate(self):
        """q, k, v each [B, H, N, D] (uint16)."""
        return tuple(np.ascontiguousarray(t.transpose(0, 2, 1, 3)) for t in (self.q, self.k, self.v))

    def in_layout(self, layout: int):
        """(qkv_or_q, k, v) arrays as the library expects them for `layout`."""
        if layout == LAYOUT_PACKED:
            return self.packed(), None, None
        if layout == LAYOUT_SEPARATE:
            return self.separate()
        raise ValueError(f"unknown layout {layout}")


def gamma_vectors(wl: Workload) -> np.ndarray:
    """Fixed per-channel scales in [0.5, 2] for Q, K, V: float32 [3, H*D].

    Drawn once from the workload's aux seed and shared by all its layers,
    standing in for a LayerNorm weight in front of the QKV projection.
    """
    rng = np.random.Generator(np.random.PCG64(wl.aux_seed))
    return rng.uniform(0.5, 2.0, size=(3, wl.H * wl.D)).astype(np.float32)


def make_layer(wl: Workload, layer: int, *, B: int | None = None, N: int | None = None,
               H: int | None = None, fmt: str = "bf16") -> LayerInputs:
    """Draw one layer's inputs for workload `wl`.

    `B`, `N`, `H` override the workload's sizes (for reduced-size parity cases
    with the same value recipe).  `fmt` is the 16-bit format the float32
    draws are rounded to: "bf16" (the workloads' own) or "f16"; the draws are
    the same for both.

    Recipes:
      iid    : Q, K, V i.i.d. N(0, 1).
      gamma  : Q, K, V = z * gamma[h*D + d], z ~ N(0, 1), gamma from gamma_vectors().
      stress : Q, K ~ N(0, 2.8^2) so that logits have std ~8 at scale 1/sqrt(D);
               V ~ N(0, 1). In every (b, h), round(0.1*N) distinct query rows i
               get one uniformly chosen key j added: Q_i <- round(Q_i + K_j),
               which makes that key dominate row i (near one-hot softmax).
    """
    B = wl.B if B is None else B
    N = wl.N if N is None else N
    H = wl.H if H is None else H
    D = wl.D
    rng = np.random.Generator(np.random.PCG64(wl.seed(layer)))
    shape = (B, N, H, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if wl.kind == "iid":
        pass
    elif wl.kind == "gamma":
        g = gamma_vectors(wl)[:, : H * D].reshape(3, 1, 1, H, D)
        q = q * g[0]
        k = k * g[1]
        v = v * g[2]
    elif wl.kind == "stress":
        q = q * np.float32(2.8)
        k = k * np.float32(2.8)
    else:
        raise ValueError(f"unknown recipe {wl.kind}")
    rnd, wid = ROUND[fmt], WIDEN[fmt]
    qb = rnd(q)
    kb = rnd(k)
    vb = rnd(v)
    if wl.kind == "stress":
        n_boost = int(round(0.1 * N))
        if n_boost > 0:
            rows = np.argsort(rng.random((B, H, N)), axis=-1)[..., :n_boost]  # [B,H,n_boost]
            keys = rng.integers(0, N, size=(B, H, n_boost))
            bi = np.arange(B)[:, None, None]
            hi = np.arange(H)[None, :, None]
            qf = wid(qb)
            kf = wid(kb)
            boosted = qf[bi, rows, hi, :] + kf[bi, keys, hi, :]
            qf[bi, rows, hi, :] = boosted
            qb = rnd(qf)
    return LayerInputs(qb, kb, vb)
