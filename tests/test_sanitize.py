"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C oracle (oracle/dsc_oracle.c) is built instrumented, and the oracle pin
  suites (tests/test_oracle_*.py, every `-m "not gpu"` test that exercises the
  oracle's arithmetic) run against that build in a child process with the
  sanitizer runtimes preloaded. Any out-of-bounds access, use after free or
  undefined operation (signed overflow, bad shift, misaligned access) aborts the
  child, and the test fails with its report.
* The low-rank launch plan (csrc/lowrank_plan.hpp), the host logic that sizes
  every matrix-core launch and the workspace, is built instrumented the same way
  and evaluated on shapes from tiny to the largest the API accepts.

The planted-mistake tests are left out of the child run: they load mutated,
uninstrumented copies of the oracle on purpose.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not available")
    return path


def _san_env(extra=None) -> dict:
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra or {})
    return env


@pytest.fixture(scope="module")
def gcc():
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc/g++ not available")


def test_oracle_pins_under_sanitizers(gcc, tmp_path):
    sys.path.insert(0, ROOT)
    import oracle

    lib = oracle.build(force=True, out=str(tmp_path / "liboracle_san.so"), extra_flags=SAN_FLAGS)
    preload = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    tests = sorted(os.path.join(HERE, f) for f in os.listdir(HERE) if f.startswith("test_oracle_") and f.endswith(".py"))
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", "not planted_mistake", *tests]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=900,
                       env=_san_env({"LD_PRELOAD": preload, "DSC_ORACLE_LIB": lib}))
    tail = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, f"oracle pins under ASan/UBSan failed (rc {r.returncode}):\n{tail}"
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    assert " passed" in r.stdout, tail


def test_launch_plan_under_sanitizers(gcc, tmp_path):
    sys.path.insert(0, HERE)
    from test_plan import build_probe

    exe = build_probe(str(tmp_path), SAN_FLAGS)
    shapes = [(1, 1, 8, 8, 1), (8, 4096, 2048, 32, 4), (1, 65536, 4096, 64, 8), (1, 2 ** 24 + 16, 16, 32, 4),
              (2 ** 24, 1, 64, 32, 4), (2 ** 31, 8, 8, 128, 8), (1, 2 ** 31, 8, 8, 8), (3, 1000, 200, 16, 3),
              (2, 77, 2 ** 24, 128, 8), (1, 2 ** 27 - 300, 8, 8, 2)]
    for B, T, D, R, W in shapes:
        for bf16 in (0, 1):
            r = subprocess.run([exe, str(B), str(T), str(D), str(R), str(W), str(bf16)], capture_output=True,
                               text=True, env=_san_env())
            assert r.returncode == 0 and "runtime error" not in r.stderr, (B, T, D, R, W, bf16, r.stderr)
