"""The host layer and the C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
and driven on the CPU.

* `sanitize/host_driver.cpp` links `fp4_api.cpp` (the C-ABI's validation, routing and
  workspace logic) against stub launchers and calls every entry point with valid, edge
  and invalid arguments; the device pointers are fake, so any host-side dereference of
  one is a sanitizer report.
* `sanitize/oracle_driver.c` runs every grid, the four quantize kinds on ties, signed
  zeros, subnormals and out-of-range values, and the exact-sum search at its bucket
  extremes.

A planted heap overflow (built with AddressSanitizer alone, so that its report and not
UBSan's object-size check names it) and a planted signed overflow (UBSan alone) show that
both sanitizers are live with these compilers and flags: a silent one would pass anything.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)


def _build(cmd):
    r = _run(cmd)
    assert r.returncode == 0, r.stderr[-4000:]


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return tmp_path_factory.mktemp("san")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(outdir):
    exe = str(outdir / "oracle_san")
    _build(["gcc", *SAN, "-ffp-contract=off", "-fopenmp", os.path.join(ROOT, "oracle", "fp4_oracle.c"),
            os.path.join(HERE, "sanitize", "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr, r.stdout[-2000:] + r.stderr[-4000:]
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")
def test_host_layer_under_sanitizers(outdir):
    exe = str(outdir / "host_san")
    _build([CLANG, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            os.path.join(ROOT, "bit_floating_point_amd", "csrc", "fp4_api.cpp"),
            os.path.join(HERE, "sanitize", "host_driver.cpp"), "-o", exe, "-rtlib=compiler-rt", "-unwindlib=libgcc"])
    r = _run([exe], env=ENV)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr, r.stdout[-2000:] + r.stderr[-4000:]
    assert "all statuses as expected" in r.stdout


PLANTED = {
    "heap": ("int main(int c,char**v){(void)v;volatile int*p=(volatile int*)__builtin_malloc(4*sizeof(int));"
             "p[3+c]=1;int s=p[3];__builtin_free((void*)p);return s;}", "address", "heap-buffer-overflow"),
    "signed": ("int main(int c,char**v){(void)v;int x=2147483647-1+c;return x+c>0;}", "undefined", "signed integer overflow"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
@pytest.mark.parametrize("case", sorted(PLANTED))
def test_planted_errors_are_reported(outdir, case):
    src, kind, want = PLANTED[case]
    c = outdir / f"planted_{case}.c"
    c.write_text(src)
    exe = str(outdir / f"planted_{case}")
    flags = [f for f in SAN if not f.startswith("-fsanitize=")] + [f"-fsanitize={kind}"]
    _build(["gcc", *flags, str(c), "-o", exe])
    r = _run([exe], env=ENV)
    assert r.returncode != 0 and want in r.stderr, r.stderr[-2000:]
