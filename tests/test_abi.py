"""The C ABI on the CPU: the library loads, exports every function that
include/vitattn.h declares, and rejects bad arguments on the host before any
device call.  No call here reaches a kernel launch: every argument set is
either invalid or an empty problem, both of which return before HIP is used.
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vitattn.h")

A = 0x7f0000000000  # fake, 16-byte aligned "device" addresses: never dereferenced
OUT = 0x7f1000000000


@pytest.fixture(scope="module")
def va():
    import vit_self_attention_amd
    return vit_self_attention_amd


def _declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vitattn_[a-z_]+)\s*\(", text)))


def _declared_enums():
    with open(HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(VITATTN_\w+)\s*=\s*(-?\d+)", text)}


def test_exports_every_declared_function(va):
    declared = _declared_functions()
    assert declared == sorted(va.EXPORTED)
    lib = ctypes.CDLL(va.LIBRARY)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_codes_match_header(va):
    enums = _declared_enums()
    for name, value in enums.items():
        if name.startswith("VITATTN_ERR_") or name == "VITATTN_OK":
            assert getattr(va._binding, name[len("VITATTN_"):]) == value, name
    assert enums["VITATTN_LAYOUT_SEPARATE_BHND"] == va.LAYOUT_SEPARATE
    assert enums["VITATTN_LAYOUT_PACKED_BN3HD"] == va.LAYOUT_PACKED


def test_version_and_strerror(va):
    assert va.version() == 200
    for name, code in _declared_enums().items():
        if name.startswith("VITATTN_ERR_"):
            msg = va.strerror(code)
            assert msg and msg != "unknown status"
    assert va.strerror(12345) == "unknown status"
    assert va.strerror(0) == "success"


def _call(va, q=A, k=None, v=None, out=OUT, B=2, H=3, N=197, D=64, scale=0.125,
          layout=None):
    if layout is None:
        layout = va.LAYOUT_PACKED if k is None else va.LAYOUT_SEPARATE
    return va.fwd_raw(q, k, v, out, B, H, N, D, scale, layout, None)


@pytest.mark.parametrize("D", [0, 1, 32, 63, 65, 71, 80, 96, 128, -64])
def test_unsupported_head_dim(va, D):
    assert _call(va, D=D) == va._binding.ERR_UNSUPPORTED_D


@pytest.mark.parametrize("bhn", [(-1, 1, 1), (1, -1, 1), (1, 1, -1)])
def test_negative_sizes(va, bhn):
    B, H, N = bhn
    assert _call(va, B=B, H=H, N=N) == va._binding.ERR_BAD_SIZE


@pytest.mark.parametrize("scale", [math.nan, math.inf, -math.inf])
def test_non_finite_scale(va, scale):
    assert _call(va, scale=scale) == va._binding.ERR_BAD_SCALE


def test_null_pointers(va):
    e = va._binding.ERR_NULL_POINTER
    assert _call(va, q=0) == e
    assert _call(va, out=0) == e
    sep = va.LAYOUT_SEPARATE
    assert _call(va, k=A + 4096, v=None, layout=sep) == e
    assert _call(va, k=None, v=A + 4096, layout=sep) == e


def test_bad_layout(va):
    e = va._binding.ERR_BAD_LAYOUT
    assert _call(va, layout=2) == e
    assert _call(va, layout=-1) == e
    # k / v must be NULL with the packed layout
    assert _call(va, k=A + 2 ** 30, v=A + 2 ** 31, layout=va.LAYOUT_PACKED) == e


def test_misaligned(va):
    e = va._binding.ERR_MISALIGNED
    assert _call(va, q=A + 2) == e
    assert _call(va, out=OUT + 8) == e
    sep = va.LAYOUT_SEPARATE
    assert _call(va, k=A + 2 ** 30 + 4, v=A + 2 ** 31) == e
    assert _call(va, k=A + 2 ** 30, v=A + 2 ** 31 + 2, layout=sep) == e


def test_overlap(va):
    e = va._binding.ERR_OVERLAP
    B, H, N, D = 2, 3, 197, 64
    t_bytes = B * H * N * D * 2
    # packed: out inside the qkv buffer (3 * t_bytes long)
    assert _call(va, out=A + 2 * t_bytes, B=B, H=H, N=N, D=D) == e
    assert _call(va, out=A - t_bytes + 16, B=B, H=H, N=N, D=D) == e
    # separate: out overlapping v
    kk, vv = A + 2 ** 30, A + 2 ** 31
    assert _call(va, k=kk, v=vv, out=vv + 1024, B=B, H=H, N=N, D=D) == e


def test_too_large(va):
    assert _call(va, B=2 ** 30, H=2 ** 10, N=2 ** 10) == va._binding.ERR_TOO_LARGE


@pytest.mark.parametrize("bhn", [(0, 3, 7), (2, 0, 7), (2, 3, 0), (0, 0, 0)])
def test_empty_problem_is_a_noop(va, bhn):
    """Empty problems return success without touching the device (the
    addresses passed here are not valid device memory)."""
    B, H, N = bhn
    assert _call(va, B=B, H=H, N=N) == va.OK
    assert _call(va, k=A + 2 ** 30, v=A + 2 ** 31, B=B, H=H, N=N) == va.OK
    # a zero-element tensor has no storage: NULL pointers are accepted then
    assert _call(va, q=0, out=0, B=B, H=H, N=N) == va.OK
    # but the other arguments are still checked
    assert _call(va, q=0, out=0, B=B, H=H, N=N, D=80) == va._binding.ERR_UNSUPPORTED_D


def test_vectorcall_module_matches_ctypes_statuses(va):
    """The vectorcall module built beside the library is the binding's
    fwd_c, and returns what the ctypes function returns for every argument
    check (none of these calls reaches the device)."""
    from vit_self_attention_amd import _vitattn_ext

    assert va.fwd_c is _vitattn_ext.vitattn_fwd
    kk, vv = A + 2 ** 30, A + 2 ** 31
    cases = [
        (A, None, None, OUT, 2, 3, 197, 65, 0.125, 1, None),           # unsupported D
        (A, None, None, OUT, -1, 3, 197, 64, 0.125, 1, None),          # negative B
        (A, None, None, OUT, 2, 3, 197, 64, math.nan, 1, None),        # NaN scale
        (None, None, None, OUT, 2, 3, 197, 64, 0.125, 1, None),        # NULL input
        (A, None, None, OUT, 2, 3, 197, 64, 0.125, 2, None),           # bad layout
        (A + 2, None, None, OUT, 2, 3, 197, 64, 0.125, 1, None),       # misaligned
        (A, kk, vv, vv + 1024, 2, 3, 197, 64, 0.125, 0, None),         # out overlaps v
        (A, None, None, OUT, 2 ** 30, 2 ** 10, 2 ** 10, 64, 0.125, 1, None),  # too large
        (A, None, None, OUT, 0, 3, 7, 64, 0.125, 1, None),             # empty: no-op
        (0, None, None, 0, 2, 3, 0, 64, 0.125, 1, 0),                  # empty, NULL stream 0
    ]
    for args in cases:
        want = va._binding.lib.vitattn_fwd(*[x if x else None for x in args[:4]], *args[4:10],
                                           args[10] or None)
        assert _vitattn_ext.vitattn_fwd(*args) == want, args
    assert _vitattn_ext.vitattn_fwd(*cases[0]) == va._binding.ERR_UNSUPPORTED_D


def test_vectorcall_module_rejects_bad_python_arguments(va):
    from vit_self_attention_amd import _vitattn_ext as ext

    good = (A, None, None, OUT, 2, 3, 197, 65, 0.125, 1, None)
    with pytest.raises(TypeError):
        ext.vitattn_fwd(*good[:10])
    with pytest.raises(TypeError):
        ext.vitattn_fwd(*good, None)
    with pytest.raises(TypeError):
        ext.vitattn_fwd("0x10", *good[1:])
    with pytest.raises(TypeError):
        ext.vitattn_fwd(*good[:4], 2.0, *good[5:])
    with pytest.raises(TypeError):
        ext.vitattn_fwd(*good[:8], "0.125", *good[9:])
    with pytest.raises(OverflowError):
        ext.vitattn_fwd(*good[:6], 2 ** 31, *good[7:])
    with pytest.raises(OverflowError):
        ext.vitattn_fwd(-1, *good[1:])
    # a float scale may arrive as an int
    assert ext.vitattn_fwd(*good[:8], 1, *good[9:]) == va._binding.ERR_UNSUPPORTED_D


def test_python_wrapper_rejects_cpu_tensors(va):
    import torch
    x = torch.zeros(1, 4, 3, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        va.fwd(x)
    # the prepared-call helper runs the same checks, and needs an output
    with pytest.raises(ValueError):
        va.fwd_args(x, out=None)
    with pytest.raises(TypeError):
        va.fwd_args(x, out=torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16))


# ---- plans (recorded call sequences).  Every case below fails a host-side
# check, or records only empty problems, so no HIP call is made.

def _plan(va, layers=3, q=None, k=None, v=None, out=None, B=2, H=3, N=197, D=64, scale=0.125,
          layout=None):
    step = 2 ** 26
    if q is None:
        q = [A + l * step for l in range(layers)]
    if out is None:
        out = [OUT + l * step for l in range(layers)]
    if layout is None:
        layout = va.LAYOUT_PACKED if k is None else va.LAYOUT_SEPARATE
    return va.plan_create_raw(q, k, v, out, B, H, N, D, scale, layout)


def test_plan_rejects_bad_arguments_before_recording(va):
    b = va._binding
    assert _plan(va, layers=0, q=[], out=[])[0] == b.ERR_BAD_SIZE
    rc, handle = _plan(va, D=80)
    assert rc == b.ERR_UNSUPPORTED_D and handle is None
    assert _plan(va, scale=math.nan)[0] == b.ERR_BAD_SCALE
    assert _plan(va, layout=7)[0] == b.ERR_BAD_LAYOUT
    # one bad call anywhere in the sequence rejects the whole plan
    q = [A, A + 2 ** 26, A + 2 * 2 ** 26 + 2]
    assert _plan(va, q=q)[0] == b.ERR_MISALIGNED
    out = [OUT, A + 2 ** 26 + 64, OUT + 2 * 2 ** 26]  # call 1 writes into its own input
    assert _plan(va, out=out)[0] == b.ERR_OVERLAP
    out = [OUT, 0, OUT + 2 * 2 ** 26]
    assert _plan(va, out=out)[0] == b.ERR_NULL_POINTER
    # separate layout needs k and v arrays; packed takes none
    sep = va.LAYOUT_SEPARATE
    assert _plan(va, layout=sep)[0] == b.ERR_NULL_POINTER
    kk = [A + 2 ** 30 + l * 2 ** 26 for l in range(3)]
    assert _plan(va, k=kk, v=kk, layout=va.LAYOUT_PACKED)[0] == b.ERR_BAD_LAYOUT


def test_plan_null_handle_arguments(va):
    lib = va._binding.lib
    arr = (ctypes.c_void_p * 1)(A)
    out = (ctypes.c_void_p * 1)(OUT)
    assert lib.vitattn_plan_create(None, 1, arr, None, None, out, 1, 1, 8, 64, 0.125,
                                   va.LAYOUT_PACKED) == va._binding.ERR_NULL_POINTER
    assert va.plan_launch_raw(None, None) == va._binding.ERR_NULL_POINTER
    assert va.plan_destroy_raw(None) == va.OK


def test_plan_of_empty_problems_records_nothing(va):
    """A plan whose calls are all empty problems holds no graph: creating,
    launching and destroying it touch no device (the addresses are fake)."""
    for bhn in [(0, 3, 7), (2, 0, 7), (2, 3, 0)]:
        rc, handle = _plan(va, B=bhn[0], H=bhn[1], N=bhn[2])
        assert rc == va.OK and handle
        assert va.plan_launch_raw(handle, None) == va.OK
        assert va.plan_destroy_raw(handle) == va.OK


# ---- the benchmark's MFMA throughput probe (include/vitattn_probe.h)

PROBE_HEADER = os.path.join(ROOT, "include", "vitattn_probe.h")


def _probe_lib():
    from vit_self_attention_amd import build
    lib = ctypes.CDLL(build.PROBE_LIBRARY)
    lib.vitattn_probe_mfma_loop.restype = ctypes.c_int
    lib.vitattn_probe_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p]
    lib.vitattn_probe_mfma_loop_flops.restype = ctypes.c_double
    lib.vitattn_probe_mfma_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    return lib


def test_probe_library_exports_every_declared_function():
    with open(PROBE_HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(vitattn_probe_[a-z_]+)\s*\(", text)))
    assert declared == ["vitattn_probe_mfma_loop", "vitattn_probe_mfma_loop_flops"]
    lib = _probe_lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_probe_argument_checks_and_flop_count():
    lib = _probe_lib()
    assert lib.vitattn_probe_mfma_loop(None, 8, 8, 1, None) == -1
    assert lib.vitattn_probe_mfma_loop(OUT, 0, 8, 1, None) == -2
    assert lib.vitattn_probe_mfma_loop(OUT, 8, 0, 1, None) == -2
    # 4 waves x 4 chains x iters MFMAs of 2*32*32*16 flops per block
    assert lib.vitattn_probe_mfma_loop_flops(3, 5) == 3 * 4 * 5 * 4 * 2 * 32 * 32 * 16


# ---- vitattn_linear argument checks (all fail before any HIP call)

def _lin(va, x=A, w=A + 2 ** 30, bias=None, residual=None, out=OUT, M=64, K=128, Nout=64, flags=0):
    return va.linear_raw(x, w, bias, residual, out, M, K, Nout, flags, None)


def test_linear_argument_checks(va):
    b = va._binding
    assert _lin(va, flags=4) == b.ERR_BAD_LAYOUT
    assert _lin(va, M=-1) == b.ERR_BAD_SIZE
    assert _lin(va, K=-32) == b.ERR_BAD_SIZE
    for K in (0, 16, 100, 1150):
        assert _lin(va, K=K) == b.ERR_UNSUPPORTED_SHAPE, K
    for Nout in (4, 12, 1001):
        assert _lin(va, Nout=Nout) == b.ERR_UNSUPPORTED_SHAPE, Nout
    assert _lin(va, x=0) == b.ERR_NULL_POINTER
    assert _lin(va, w=0) == b.ERR_NULL_POINTER
    assert _lin(va, out=0) == b.ERR_NULL_POINTER
    assert _lin(va, x=A + 8) == b.ERR_MISALIGNED
    assert _lin(va, bias=A + 2 ** 31 + 4) == b.ERR_MISALIGNED
    assert _lin(va, residual=OUT + 2 ** 31 + 2) == b.ERR_MISALIGNED
    assert _lin(va, M=2 ** 21, K=1024) == b.ERR_TOO_LARGE  # x spans 4 GiB
    # out overlapping x, w or bias; a residual shifted against out
    assert _lin(va, out=A + 256) == b.ERR_OVERLAP
    assert _lin(va, out=A + 2 ** 30 + 64) == b.ERR_OVERLAP
    assert _lin(va, bias=OUT + 64) == b.ERR_OVERLAP
    assert _lin(va, residual=OUT + 128) == b.ERR_OVERLAP


def test_linear_empty_is_a_noop(va):
    assert _lin(va, M=0) == va.OK
    assert _lin(va, Nout=0) == va.OK
    assert _lin(va, M=0, x=0, out=0) == va.OK


def test_fwd_shape_describes_the_launch_without_a_device(va):
    """vitattn_fwd_shape on the CPU (no device: the compute-unit count is
    unknown, so no workgroup loops; 256 compute units are assumed): the
    split-key choice on grids that four-wave items would leave
    underfilled, and otherwise the largest wave count that still gives 128
    workgroups (half the compute units)."""
    cases = {
        # (B, H, N, D): (waves, split_keys, items)
        (1, 12, 197, 64): (4, True, 12 * 7),     # 4 key tiles, 84 blocks of 32 queries
        (3, 12, 101, 64): (4, True, 36 * 4),     # 2 key tiles
        (2, 16, 256, 72): (4, True, 32 * 8),     # 4 key tiles
        (1, 1, 64, 72): (1, False, 2),           # one key tile: never split
        (1, 1, 729, 72): (4, True, 23),          # 12 key tiles, tiny grid: split, 3 tiles a wave
        (1, 12, 577, 64): (4, True, 12 * 19),    # 4 waves would give 60 < 128 workgroups
        (2, 16, 257, 64): (4, True, 32 * 9),     # 5 key tiles, 96 four-wave items
        (1, 16, 729, 72): (4, True, 16 * 23),
        (1, 1, 8192, 64): (2, False, 128),       # 256 blocks of 32: past the split's bounds
        (1, 4, 64, 64): (1, False, 4 * 2),       # one key tile: never split
        (8, 16, 257, 64): (4, False, 128 * 3),
        (4, 16, 729, 72): (4, False, 64 * 6),
        (6, 16, 729, 72): (4, False, 96 * 6),
        (48, 16, 729, 72): (4, False, 768 * 6),
        (64, 16, 256, 72): (4, False, 1024 * 2),  # items of 128 fill the chip: not split
        (8, 16, 256, 72): (4, False, 128 * 2),    # 256 items of 128, one per compute unit
        (4, 16, 256, 72): (4, True, 64 * 8),      # 128 items of 128 would leave half idle
    }
    for (B, H, N, D), (waves, split, items) in cases.items():
        got = va.fwd_shape(B, H, N, D)
        assert (got["waves"], got["split_keys"], got["items"]) == (waves, split, items), (B, H, N, D)
        assert got["workgroups"] == items and not got["looping"]
    for bad, code in (((1, 1, 8, 80), va._binding.ERR_UNSUPPORTED_D),
                      ((-1, 1, 8, 64), va._binding.ERR_BAD_SIZE),
                      ((1 << 20, 1 << 10, 1 << 10, 64), va._binding.ERR_TOO_LARGE)):
        with pytest.raises(va.VitAttnError) as e:
            va.fwd_shape(*bad)
        assert e.value.status == code
    rc = va._binding.lib.vitattn_fwd_shape(1, 1, 8, 64, 7, None, None, None, None)
    assert rc == va._binding.ERR_NULL_POINTER
    i = ctypes.c_int()
    rc = va._binding.lib.vitattn_fwd_shape(1, 1, 8, 64, 7, *[ctypes.byref(i)] * 4)
    assert rc == va._binding.ERR_BAD_LAYOUT
