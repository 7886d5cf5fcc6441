"""Host sanitizer tier: the library's argument validation and launch planning (csrc/plan.cpp,
pure C++) built alone with g++ and AddressSanitizer + UndefinedBehaviorSanitizer into the fuzz
driver tests/plan_fuzz.cpp, which checks seeded random and extreme kata_problem values (sizes,
dtypes, layouts, groups, eps, strides) against the documented contracts.  CPU only; skipped
when g++ is not installed."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kernelized_psd_feature_amd", "csrc")


@pytest.fixture(scope="module")
def fuzz_driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path_factory.mktemp("plan_fuzz") / "plan_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "plan_fuzz.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2026])
def test_validation_and_planning_are_clean_under_sanitizers(fuzz_driver, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([fuzz_driver, str(seed), "200000"], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.startswith("ok 200000 problems")
    counts = [int(x) for x in r.stdout.replace(",", " ").split() if x.isdigit()][1:]
    assert all(c > 1000 for c in counts), r.stdout          # every form saw valid problems
