"""The host side of libstc (argument validation, cyclic Jacobi, water-filling
and its variants, Lloyd, quantizer steps) built with the address and
undefined-behaviour sanitizers (g++, host code only; the kernel launchers are
stubs that report failure) and driven through the C ABI: the sanitizers must
stay silent, and the answers must equal the oracle's."""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import codec, rht

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    hip_lib = os.path.join(ROCM, "lib", "libamdhip64.so")
    if not gxx or not os.path.exists(hip_lib):
        pytest.skip("g++ or the HIP runtime library is missing")
    out = str(tmp_path_factory.mktemp("asan") / "host_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           os.path.join(ROOT, "spectral_transform_codec_amd", "csrc", "stc_host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "kernel_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
           "-L" + os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def run(driver, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout.splitlines()


def fmt(a):
    return " ".join(repr(float(v)) for v in np.asarray(a, np.float64).ravel())


def test_sanitized_host_math_matches_oracle(driver):
    rng = np.random.default_rng(60)
    lines, checks = [], []
    for b in range(0, 10):
        lines.append(f"ds {b}")
        checks.append(("ds", b))
    for avg in (0.1, 1.33, 2.0, 4.0, 8.0):
        lines.append(f"tb {avg} 128")
        checks.append(("tb", avg))
    for trial in range(12):
        d = int(rng.integers(1, 129))
        lam = rng.lognormal(0, 2, d)
        if trial % 3 == 0:
            lam[rng.integers(0, d, 2)] = 0.0
        B = int(rng.integers(0, 8 * d + 1))
        lines.append(f"wf {d} {B} {fmt(lam)}")
        checks.append(("wf", lam, B))
    lam = np.sort(rng.lognormal(0, 1.5, 128))[::-1]
    for variant, vid, param in (("operational", 1, 0.0), ("grouped", 2, 4.0), ("floor", 3, 1.0), ("gap", 4, 20.0)):
        lines.append(f"al 128 256 {vid} {param} {fmt(lam)}")
        checks.append(("al", lam, 256, variant, param))
    for d in (1, 2, 8, 37, 128):
        a = rng.standard_normal((d, d))
        a = a @ a.T / d
        lines.append(f"eh {d} {fmt(a)}")
        checks.append(("eh", a))
    smp = rng.standard_normal(4000) * 0.1
    lines.append(f"lm {smp.size} 8 1e-12 10000 {fmt(smp)}")
    checks.append(("lm", smp))
    lines.append("inv")
    out = run(driver, lines)
    k = 0
    for c in checks:
        vals = out[k].split()
        k += 1
        if c[0] == "ds":
            got = float(vals[0])
            want = codec.delta_star(c[1]) if 1 <= c[1] <= 8 else float("nan")
            assert (math.isnan(got) and math.isnan(want)) or abs(got - want) <= 1e-12 * want
        elif c[0] == "tb":
            assert int(vals[0]) == codec.total_bits_for(c[1], 128)
        elif c[0] == "wf":
            assert int(vals[0]) == 0
            assert np.array_equal(np.array(vals[1:], np.int64), codec.water_fill(c[1], c[2]))
        elif c[0] == "al":
            assert int(vals[0]) == 0
            assert np.array_equal(np.array(vals[1:], np.int64), codec.allocate_bits(c[1], c[2], c[3], c[4]))
        elif c[0] == "eh":
            a = c[1]
            d = a.shape[0]
            assert int(vals[0]) == 0
            lam_g = np.array(vals[1:1 + d], np.float64)
            u_g = np.array(vals[1 + d:], np.float64).reshape(d, d)
            u_o, lam_o = codec.eigenbasis(a)
            assert np.abs(lam_g - lam_o).max() <= 1e-12 * max(1.0, abs(lam_o).max())
            assert np.abs(u_g - u_o).max() <= 1e-8
        elif c[0] == "lm":
            assert int(vals[0]) == 0
            cg = np.array(vals[2:], np.float64)
            co, _ = rht.lloyd_max(c[1])
            assert np.abs(cg - co).max() <= 1e-9
    inv = [int(v) for v in out[k].split()]
    assert all(s < 0 for s in inv), inv
    assert out[k + 1] == "1"
