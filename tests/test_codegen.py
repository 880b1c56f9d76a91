"""Properties of the compiled gfx950 code that the kernel's correctness or
speed relies on, checked on the device assembly hipcc writes for it (CPU
only: the kernel source is compiled with the library's own flags, nothing
runs on a GPU).

* The direct-to-LDS fetches are written as inline asm that sets M0 itself.
  That is only safe while nothing else in the kernel uses M0: every M0
  write must be one of those fetch sequences, with the wait state the
  hardware needs between the write and the fetch.
* No kernel may spill to scratch memory, and the four-wave kernels must
  fit two waves per SIMD (at most 256 registers, VGPRs and AGPRs together).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vit_self_attention_amd", "csrc")

pytestmark = pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def _compile(tmp_path_factory, source):
    from vit_self_attention_amd import build as b
    out = tmp_path_factory.mktemp("codegen") / (source + ".s")
    flags = [f for f in b.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [b.HIPCC, *flags, "-S", "--cuda-device-only", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", str(out), os.path.join(CSRC, source)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return out.read_text()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return _compile(tmp_path_factory, "vitattn_fwd.hip")


@pytest.fixture(scope="module")
def linear_asm(tmp_path_factory):
    return _compile(tmp_path_factory, "vitattn_linear.hip")


def _kernels(text, kind="fwd_kernel"):
    """{kernel symbol: (body instruction lines, metadata tail)}"""
    out = {}
    for m in re.finditer(r"^(_Z\S*" + kind + r"\S*):[ \t]*(?:;.*)?$", text, re.M):
        end = text.index(".Lfunc_end", m.end())
        body = [ln.strip() for ln in text[m.end():end].splitlines()]
        body = [ln.split(";")[0].strip() for ln in body if ln and not ln.startswith((";", "."))]
        out[m.group(1)] = (body, text[end:end + 4000])
    return out


def test_every_kernel_instantiation_found(asm):
    names = list(_kernels(asm))
    # D in {64, 72} x (NW in {1, 2, 4} without split, NW = 4 with split of
    # one tile a wave, and of several) x element format {bf16, fp16}
    assert len(names) == 20, names


def test_m0_is_only_written_by_the_fetch_sequence(asm):
    for name, (body, _) in _kernels(asm).items():
        for i, ln in enumerate(body):
            if "m0" not in ln:
                continue
            # the only instruction that names m0 is the asm's own write ...
            assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", ln), (name, ln)
            # ... followed by the wait state and the fetch that reads it
            assert body[i + 1] == "s_nop 0", (name, body[i:i + 3])
            assert body[i + 2].startswith("global_load_lds_dwordx4"), (name, body[i:i + 3])
        fetches = [ln for ln in body if ln.startswith("global_load_lds")]
        writes = [ln for ln in body if ln.startswith("s_mov_b32 m0")]
        assert len(fetches) == len(writes) > 0, name


def test_no_scratch_and_two_waves_per_simd(asm):
    for name, (_, meta) in _kernels(asm).items():
        scratch = int(re.search(r"ScratchSize: (\d+)", meta).group(1))
        total = int(re.search(r"TotalNumVgprs: (\d+)", meta).group(1))
        assert scratch == 0, (name, scratch)
        nw = int(re.search(r"fwd_kernelILi\d+ELi(\d+)E", name).group(1))
        if nw == 4:
            assert total <= 256, (name, total)


def test_linear_kernels_m0_and_registers(linear_asm):
    """The linear kernels use the same direct-to-LDS fetch sequence, spill
    nothing and fit two waves per SIMD."""
    ks = _kernels(linear_asm, "linear_kernel")
    # four tile shapes x {bf16, fp16}, and the largest with streaming stores too
    assert len(ks) == 10, list(ks)
    for name, (body, meta) in ks.items():
        for i, ln in enumerate(body):
            if "m0" in ln:
                assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", ln), (name, ln)
                assert body[i + 1] == "s_nop 0" and body[i + 2].startswith("global_load_lds_dwordx4")
        assert int(re.search(r"ScratchSize: (\d+)", meta).group(1)) == 0, name
        assert int(re.search(r"TotalNumVgprs: (\d+)", meta).group(1)) <= 256, name


def test_small_division_is_exact_over_its_range():
    """The kernels divide item and head indices with div_small:
    floor(fma(n, rcp(d), 2^-12)) in fp32, for 0 <= n < 2048 and
    1 <= d < 2048 (fewer than 2048 items).  Checked here for every such n
    and d, with the reciprocal correctly rounded and up to two ulp either
    side of 1/d (v_rcp_f32 is accurate to one ulp), the fma rounded once."""
    import numpy as np
    n = np.arange(0, 2048, dtype=np.int64)
    nf = n.astype(np.float64)
    for d in range(1, 2048):
        r0 = np.float32(1.0) / np.float32(d)
        rs = [r0]
        lo = hi = r0
        for _ in range(2):
            lo = np.nextafter(lo, np.float32(0), dtype=np.float32)
            hi = np.nextafter(hi, np.float32(1), dtype=np.float32)
            rs += [lo, hi]
        for r in rs:
            # n * r is exact in float64 (24-bit by 11-bit significands); one
            # rounding of n * r + 2^-12 to fp32 is the fma
            x = (nf * np.float64(r) + 2.0 ** -12).astype(np.float32)
            q = x.astype(np.int64)  # truncation, as v_cvt_i32_f32
            assert np.array_equal(q, n // d), (d, float(r))


def test_multiplier_division_is_exact_where_launch_allows_it():
    """The split kernel divides by qblocks and H as (n * ceil(2^k / d)) >> k
    (k = 16 and 20), with the multipliers computed on the host.  That is
    n / d whenever n * d < 2^k, the condition launch checks; here for every
    such n and d (d up to 2047)."""
    import numpy as np
    for k in (16, 20):
        for d in range(1, 2048):
            n = np.arange(0, -(-(1 << k) // d), dtype=np.int64)  # n * d < 2^k
            m = -(-(1 << k) // d)
            assert np.array_equal((n * m) >> k, n // d), (k, d)
