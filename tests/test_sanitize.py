"""The host-only code under address and undefined-behaviour sanitizers.

Two drivers, built here with gcc/g++ and -fsanitize=address,undefined (any
report aborts the run):
  * tests/sanitize/host_checks.cpp drives libvitattn's host-only argument
    checks (vit_self_attention_amd/csrc/vitattn_host.cpp: every vitattn_fwd
    and vitattn_linear check, the size limits at the edge of 64-bit
    arithmetic, the kernel's launch shapes, the status strings); its output
    is compared with the status codes include/vitattn.h documents;
  * tests/sanitize/oracle_checks.c runs the C oracle (with OpenMP) on small
    cases in both layouts and both element formats, checking rows of P sum
    to 1, N = 1 gives V, the row entry point agrees with the full forward,
    and the 4-token closed form.
Neither touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-Wall", "-Werror"]

ERR = {"OK": 0, "NULL": -1, "SIZE": -2, "D": -3, "SCALE": -4, "LAYOUT": -5, "ALIGN": -6,
       "LARGE": -7, "OVERLAP": -9, "SHAPE": -11}

EXPECTED = {
    "fwd_ok_packed": "OK", "fwd_ok_separate": "OK", "fwd_ok_fp16": "OK",
    "fwd_ok_zero_scale": "OK", "fwd_empty_b": "OK", "fwd_empty_n": "OK",
    "fwd_bad_layout": "LAYOUT", "fwd_packed_with_k": "LAYOUT", "fwd_negative_b": "SIZE",
    "fwd_negative_n": "SIZE", "fwd_d80": "D", "fwd_nan_scale": "SCALE", "fwd_inf_scale": "SCALE",
    "fwd_null_out": "NULL", "fwd_null_v": "NULL", "fwd_misaligned_q": "ALIGN",
    "fwd_misaligned_k": "ALIGN", "fwd_overlap_packed": "OVERLAP",
    "fwd_overlap_separate_v": "OVERLAP", "fwd_adjacent_no_overlap": "OK",
    "fwd_huge_all": "LARGE", "fwd_huge_bh": "LARGE", "fwd_huge_n": "LARGE", "fwd_n_limit": "OK",
    "fwd_n_past_limit": "LARGE", "fwd_rows_past_2_40": "LARGE", "fwd_token_stride": "LARGE",
    "fwd_items_past_2_30": "LARGE",
    "lin_ok": "OK", "lin_ok_inplace_residual": "OK", "lin_empty": "OK", "lin_bad_flags": "LAYOUT",
    "lin_negative_m": "SIZE", "lin_k_not_32": "SHAPE", "lin_nout_not_8": "SHAPE",
    "lin_null_w": "NULL", "lin_misaligned_bias": "ALIGN", "lin_x_4gib": "LARGE",
    "lin_huge_all": "LARGE", "lin_overlap_x": "OVERLAP", "lin_shifted_residual": "OVERLAP",
}

# launch shapes on a 256-CU part (0: no device known)
SHAPES = {
    "shape_c1": "waves=4 split=1 qblocks=7 items=84 grid=84",
    "shape_c3": "waves=4 split=1 qblocks=8 items=256 grid=256",
    "shape_c4": "waves=4 split=0 qblocks=3 items=1152 grid=512",
    "shape_c5": "waves=4 split=0 qblocks=6 items=4608 grid=512",
    "shape_c5_no_device": "waves=4 split=0 qblocks=6 items=4608 grid=4608",
    "shape_384x6": "waves=4 split=0 qblocks=6 items=576 grid=512",
    "shape_384x9": "waves=4 split=0 qblocks=6 items=864 grid=512",
    "shape_n1024x4": "waves=4 split=0 qblocks=8 items=512 grid=512",
    "shape_one_token": "waves=1 split=0 qblocks=1 items=1 grid=1",
    "shape_max_n": "waves=4 split=0 qblocks=131072 items=131072 grid=512",
}


def _sanitizers_available(tmp_path):
    if not shutil.which("gcc") or not shutil.which("g++"):
        return False
    src = tmp_path / "probe.c"
    src.write_text("int main(void) { return 0; }\n")
    res = subprocess.run(["gcc", "-fsanitize=address,undefined", "-o", str(tmp_path / "probe"), str(src)],
                         capture_output=True)
    return res.returncode == 0


def _run(cmd, env=None):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, f"{' '.join(cmd)} failed ({res.returncode}):\n{res.stdout}\n{res.stderr}"
    return res.stdout


@pytest.fixture(scope="module")
def tmp(tmp_path_factory):
    t = tmp_path_factory.mktemp("sanitize")
    if not _sanitizers_available(t):
        pytest.skip("gcc with -fsanitize=address,undefined is not available")
    return t


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    return env


def test_host_checks_under_sanitizers(tmp):
    exe = str(tmp / "host_checks")
    _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
          "-I", os.path.join(ROOT, "vit_self_attention_amd", "csrc"), "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
          os.path.join(ROOT, "vit_self_attention_amd", "csrc", "vitattn_host.cpp")])
    out = _run([exe], env=_env())
    got = {}
    for line in out.splitlines():
        name, rest = line.split(" ", 1)
        got[name] = rest
    for name, code in EXPECTED.items():
        status = int(got[name].split()[0])
        assert status == ERR[code], f"{name}: {got[name]} (expected {code})"
    assert got["fwd_empty_b"].endswith("empty") and got["lin_empty"].endswith("empty")
    for name, shape in SHAPES.items():
        assert got[name] == "0 " + shape, name
    for code in range(0, 12):
        assert got[f"strerror_{code}"] not in ("", "unknown status"), code
    assert got["strerror_12"] == "unknown status"
    assert got["version"] == "200"


def test_oracle_under_sanitizers(tmp):
    exe = str(tmp / "oracle_checks")
    _run(["gcc", "-std=c11", "-fopenmp", *SAN, "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"),
          os.path.join(ROOT, "oracle", "vitattn_oracle.c"), "-lm"])
    out = _run([exe], env=_env())
    assert out.startswith("ok "), out
    assert int(out.split()[1]) > 3000
