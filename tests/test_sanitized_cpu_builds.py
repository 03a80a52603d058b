"""The oracle and the seeded input generator built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only), with the oracle's pins and
the generator's tests run against those builds in a child process.  Any
out-of-bounds access, use after free or undefined operation in either C
source aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], stdout=subprocess.PIPE, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    libs = {}
    for var, src, std in (("MOE_ORACLE_LIB", "oracle/moe_oracle.c", "-std=c11"),
                          ("MOE_SYNTH_LIB", "synthetic/synth.c", "-std=gnu11")):
        out = str(tmp_path / (os.path.basename(src)[:-2] + "_san.so"))
        subprocess.check_call(["gcc", std, "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas"] + SAN +
                              [os.path.join(ROOT, src), "-o", out, "-lm"])
        libs[var] = out
    env = dict(os.environ, **libs)
    # the sanitizer runtime must come first among the preloaded libraries; whatever is already
    # preloaded stays, after it
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"  # the interpreter itself leaks by design
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_synthetic.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    tail = r.stdout[-4000:]
    # the child really ran the sanitizer builds
    names = subprocess.run([sys.executable, "-c", "import oracle, synthetic; print(oracle.lib()._name); "
                            "print(synthetic.lib()._name)"], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                           stderr=subprocess.STDOUT, text=True, timeout=300).stdout.split()
    assert names[-2:] == [libs["MOE_ORACLE_LIB"], libs["MOE_SYNTH_LIB"]], names
    assert r.returncode == 0, tail
    assert "passed" in tail and "AddressSanitizer" not in tail and "runtime error" not in tail, tail
