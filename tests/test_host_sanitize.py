"""AddressSanitizer + UndefinedBehaviorSanitizer run of libhsq's host code.

api.cpp and host.cpp -- argument validation, error reporting, the codebook
generator and the tier plan -- are compiled with g++ -fsanitize=address,undefined
into a driver executable (tests/sanitize/abi_driver.cpp) that takes the device
code from the built libhsq.so.  The driver makes the host-only calls of
test_abi.py (codebooks and tier plans, checked here against the oracle; the
argument errors of every entry point, with the codes the C ABI states) plus
randomised tier plans with exact-size output buffers.  Any sanitizer report
fails the test.  Nothing here touches a GPU: the GPU code is not instrumented.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import codebook as ocb
from oracle import tiers as otiers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "compressed_decode_attention_turboquant_amd")
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libhsq.so")
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
CFLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *SAN, "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-Wall"]
REPORTS = ("AddressSanitizer", "LeakSanitizer", "runtime error", "UndefinedBehaviorSanitizer")


def _have_toolchain():
    gxx = shutil.which("g++")
    if not gxx:
        return False
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True)
    return os.path.isabs(asan.stdout.strip()) and os.path.exists(
        os.path.join(ROCM, "lib", "libamdhip64.so"))


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not _have_toolchain():
        pytest.skip("g++ with libasan or the HIP runtime library is not available")
    if not os.path.exists(LIB):
        pytest.skip("libhsq.so is not built")
    out = tmp_path_factory.mktemp("hsq_sanitize")
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "host.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")):
        obj = str(out / (os.path.basename(src) + ".o"))
        r = subprocess.run(["g++", *CFLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    # the host objects really are instrumented
    syms = subprocess.run(["nm", objs[0]], capture_output=True, text=True).stdout
    assert "__asan_report_" in syms and "__ubsan_handle_" in syms
    exe = str(out / "abi_driver")
    r = subprocess.run(["g++", *SAN, *objs, "-L", PKG, "-lhsq", "-L", os.path.join(ROCM, "lib"),
                        "-lamdhip64", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM}/lib", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run(exe, commands):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:strict_string_checks=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], input="\n".join(commands) + "\n", capture_output=True, text=True,
                       env=env, timeout=300)
    for word in REPORTS:
        assert word not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    return r.stdout.splitlines()


def test_argument_errors_under_sanitizers(driver):
    (line,) = run(driver, ["errors"])
    assert line.startswith("errors ") and int(line.split()[1]) >= 60


def test_codebooks_under_sanitizers(driver):
    cases = [(64, 3), (64, 4), (128, 3), (128, 4), (16, 2), (3, 3), (256, 4), (4096, 1)]
    lines = run(driver, [f"codebook {d} {b}" for d, b in cases])
    for (d, b), line in zip(cases, lines):
        head, tail = line.split("|")
        vals = head.split()
        assert vals[:2] == ["codebook", "0"]
        c = np.array(vals[2:], dtype=np.float32)
        t = np.array(tail.split(), dtype=np.float32)
        oc, ot = ocb.codebook_f32(d, b)
        np.testing.assert_array_max_ulp(c, oc, maxulp=1)
        np.testing.assert_array_max_ulp(t, ot, maxulp=1)


def _tier_cases():
    cases = [(512, 4, 32, 16, 8), (8192, 4, 64, 164, 16), (300, 4, 64, 7, 16), (50, 4, 64, 0, 8),
             (1, 4, 0, 0, 8), (1000, 0, 0, 0, 8)]
    out = []
    for T, ns, nr, nm, gn in cases:
        rng = np.random.default_rng(T + nm)
        lo, hi = ns, max(T - nr, ns)
        out.append((T, ns, nr, gn, np.sort(rng.choice(np.arange(lo, hi),
                                                      size=min(nm, max(hi - lo, 0)),
                                                      replace=False))))
    # randomised plans: marks anywhere (repeats allowed), sinks or windows
    # longer than the sequence, group sizes 1..17
    rng = np.random.default_rng(20261203)
    for _ in range(60):
        T = int(rng.integers(1, 3000))
        ns, nr = int(rng.integers(0, 40)), int(rng.integers(0, 300))
        gn = int(rng.integers(1, 18))
        nm = int(rng.integers(0, 64))
        out.append((T, ns, nr, gn, rng.integers(0, T, size=nm)))
    return out


def test_tier_plans_under_sanitizers(driver):
    cases = _tier_cases()
    cmds = [" ".join(map(str, [T, ns, nr, gn, len(m), *m.tolist()])) for T, ns, nr, gn, m in cases]
    lines = run(driver, ["tier " + c for c in cmds])
    assert len(lines) == len(cases)
    for (T, ns, nr, gn, m), line in zip(cases, lines):
        head, l1s, gps = line.split("|")
        tag, rc, n1, ng = head.split()
        assert (tag, rc) == ("tier", "0"), line
        ol1, og = otiers.tier_plan(T, ns, nr, m, gn)
        np.testing.assert_array_equal(np.array(l1s.split(), dtype=np.int64), ol1)
        np.testing.assert_array_equal(np.array(gps.split(), dtype=np.int64).reshape(-1, gn)
                                      if int(ng) else og.reshape(0, gn), og)
        assert int(n1) == len(ol1) and int(ng) == len(og)


def test_workspace_sizes_under_sanitizers(driver):
    shapes = [(1, 8, 8, 128, 10, 0, 0, 8), (2, 32, 8, 128, 40, 30, 4, 16),
              (64, 64, 8, 128, 1087, 442, 32, 16), (1, 32, 8, 64, 5000, 16000, 400, 8)]
    lines = run(driver, ["workspace " + " ".join(map(str, s)) for s in shapes])
    for line in lines:
        tag, n = line.split()
        assert tag == "workspace" and int(n) > 0 and int(n) % 256 == 0
