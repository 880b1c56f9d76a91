"""Every kernel path the launcher can pick, compared with the fp64 oracle on
every element, in bf16 and in fp16, at realistic encoder shapes.

The launcher (vitattn_fwd_shape describes its choice) picks, per problem:
  * split keys: 2..4 key tiles on a grid too small to fill the chip, four
    waves share one 32-query block and split its keys;
  * one workgroup per (image, head, query block) item with 1, 2 or 4 waves
    (32 queries per wave);
  * four-wave workgroups that loop over the items, two per compute unit,
    when there are at least twice as many items as such slots.
Each case below states the path it reaches, and the test first checks that
the launcher still picks that path for the shape, so a change of dispatch
cannot silently move a case onto another path.  The exact-result claim the
kernels are held to is the Pi0 Flash Attention tutorial's (section 1: the
fast kernel leaves the outputs unchanged; section 4.2 table).
"""
import numpy as np
import pytest

import oracle
from gpu_util import LAYOUT_PACKED, LAYOUT_SEPARATE, logical
from workloads import Workload, make_layer

pytestmark = pytest.mark.gpu

# bf16: the stated bar; fp16: half of it (derived in test_parity_fp16_gpu.py)
TOL = {"bf16": (2e-2, 2e-3), "f16": (1e-2, 1e-3)}

# (id, B, H, N, D, layout, recipe, expected path on a 256-CU MI355X)
#   path = (waves, split_keys, looping)
PATHS = [
    # split keys, D = 64: ViT-B/16 at 224 px (4 key tiles) and 160 px x 3 (2 tiles)
    ("split64_vitb224", 1, 12, 197, 64, LAYOUT_SEPARATE, "iid", (4, True, False)),
    ("split64_vitb160x3", 3, 12, 101, 64, LAYOUT_PACKED, "iid", (4, True, False)),
    # split keys, D = 72: SigLIP at 224 px x 2 (4 key tiles)
    ("split72_siglip224x2", 2, 16, 256, 72, LAYOUT_PACKED, "gamma", (4, True, False)),
    # split keys with many heads and several images: the first item's
    # coordinates come from multiply-shift divisions by qblocks and H (1016
    # and 747 items, H not a power of two)
    ("split64_127heads_x2", 2, 127, 100, 64, LAYOUT_SEPARATE, "iid", (4, True, False)),
    ("split72_83heads_x3", 3, 83, 96, 72, LAYOUT_PACKED, "gamma", (4, True, False)),
    # short sequences whose 128-query items give every compute unit a
    # workgroup: four waves per item, not split (8 images at N = 256)
    ("nw4_one_n256x8", 8, 16, 256, 72, LAYOUT_PACKED, "gamma", (4, False, False)),
    # split keys over more than 4 key tiles, each wave taking tiles w,
    # w + 4, ...: ViT-B/16 at 384 px, one image (10 tiles, 228 items); one
    # head at N = 729 (12 tiles, 23 items); ViT-L/14 at 224 px, two views
    # (5 tiles: wave 0 takes two); SigLIP at 384 px, one image (368 items)
    ("msplit_vitb384x1", 1, 12, 577, 64, LAYOUT_PACKED, "iid", (4, True, False)),
    ("msplit_1head_n729_d64", 1, 1, 729, 64, LAYOUT_PACKED, "stress", (4, True, False)),
    ("msplit_1head_n729_d72", 1, 1, 729, 72, LAYOUT_PACKED, "stress", (4, True, False)),
    ("msplit_vitl224x2", 2, 16, 257, 64, LAYOUT_PACKED, "iid", (4, True, False)),
    ("msplit_vitl224x2_d72", 2, 16, 257, 72, LAYOUT_SEPARATE, "iid", (4, True, False)),
    ("msplit_384x1_d72", 1, 16, 729, 72, LAYOUT_PACKED, "stress", (4, True, False)),
    # one wave per workgroup: one key tile (N = 64), four heads (8 items)
    ("nw1_n64_d64", 1, 4, 64, 64, LAYOUT_PACKED, "stress", (1, False, False)),
    ("nw1_n64_d72", 1, 4, 64, 72, LAYOUT_SEPARATE, "stress", (1, False, False)),
    # two waves per workgroup: one head at N = 8192 (256 blocks of 32, past
    # the split's bounds; 128 items)
    ("nw2_n8192_d64", 1, 1, 8192, 64, LAYOUT_PACKED, "stress", (2, False, False)),
    ("nw2_n8192_d72", 1, 1, 8192, 72, LAYOUT_PACKED, "stress", (2, False, False)),
    # four waves, one workgroup per item, fewer workgroups than slots:
    # ViT-L/14 at 224 px x 8 and 384 px x 4 (384 items each)
    ("nw4_one_vitl224x8", 8, 16, 257, 64, LAYOUT_PACKED, "iid", (4, False, False)),
    ("nw4_one_384x4_d72", 4, 16, 729, 72, LAYOUT_PACKED, "stress", (4, False, False)),
    # four waves, one workgroup per item: as many items as workgroup slots
    # (4 images, N = 1024: 512 items)
    ("nw4_one_n1024x4_d64", 4, 16, 1024, 64, LAYOUT_PACKED, "stress", (4, False, False)),
    ("nw4_one_n1024x4_d72", 4, 16, 1024, 72, LAYOUT_PACKED, "stress", (4, False, False)),
    # four-wave looping workgroups taking one or two items each: one GPU's
    # share (6 images) of the 48-image 384 px call over 8 GPUs (576 items
    # on 512 workgroups), and 9 images (864 items: a second item for the
    # younger workgroups too)
    ("loop_384x6_d64", 6, 16, 729, 64, LAYOUT_PACKED, "stress", (4, False, True)),
    ("loop_384x6_d72", 6, 16, 729, 72, LAYOUT_PACKED, "stress", (4, False, True)),
    ("loop_384x9_d72", 9, 16, 729, 72, LAYOUT_SEPARATE, "stress", (4, False, True)),
    # four-wave looping workgroups: ViT-L/14 at 224 px x 24 (1152 items) and
    # 384 px x 12 (1152 items), and a one-tile sequence (N = 64, 1536 items)
    ("loop_vitl224x24", 24, 16, 257, 64, LAYOUT_PACKED, "iid", (4, False, True)),
    ("loop_384x12_d72", 12, 16, 729, 72, LAYOUT_PACKED, "stress", (4, False, True)),
    ("loop_384x12_d64", 12, 16, 729, 64, LAYOUT_SEPARATE, "stress", (4, False, True)),
    ("loop_n64_d72", 96, 16, 64, 72, LAYOUT_PACKED, "iid", (4, False, True)),
]


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def va():
    import vit_self_attention_amd
    return vit_self_attention_amd


def _to_dev(bits, fmt, device):
    import torch
    if bits is None:
        return None
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).to(device)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("case", PATHS, ids=[p[0] for p in PATHS])
def test_path_parity(dev, va, case, fmt):
    import torch
    name, B, H, N, D, layout, kind, (waves, split, looping) = case
    shape = va.fwd_shape(B, H, N, D, layout)
    print(f"[path] {name} {fmt}: B={B} H={H} N={N} D={D} layout={layout} -> {shape}", flush=True)
    assert (shape["waves"], shape["split_keys"], shape["looping"]) == (waves, split, looping), \
        f"{name}: the launcher no longer picks the path this case is for"
    wl = Workload("t", name, B=B, N=N, H=H, D=D, layout=layout, layers=1, kind=kind,
                  index=100 + len(name))
    li = make_layer(wl, B * 7 + N, fmt=fmt)
    arrs = li.in_layout(layout)
    ts = [_to_dev(a, fmt, dev) for a in arrs]
    o = va.fwd(ts[0], ts[1], ts[2], scale=wl.scale)
    torch.cuda.synchronize(dev)
    got = logical(o, layout)
    ref = oracle.attention(*arrs, layout, B, H, N, D, wl.scale, fmt=fmt)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - ref)
    tmax, tmean = TOL[fmt]
    print(f"[path] {name} {fmt}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= tmax and err.mean() <= tmean, name
