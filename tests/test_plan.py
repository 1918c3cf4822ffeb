"""The low-rank launch plan (csrc/lowrank_plan.hpp) on the CPU: a small host program
built with g++ from the same header prints the plan for given sizes.

* The dx + dU pass with fused dz writes each sequence's fp32 dz partial [T][R]
  through one buffer resource, whose range stops at 2^31 - 1 bytes (stores past it
  are dropped by the hardware). The plan must take the separate dz pass once
  T * R * 4 passes that limit.
* Every launch of the matrix-core plan stays below a dispatch's 2^32 work-items;
  beyond, the vector-ALU kernels (grid-stride loops) take the problem.
* The workspace the library reports equals the plan's.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "dynamic_short_convolutions_amd", "csrc")
LIM = 0x7FFFFFFF


def build_probe(out_dir: str, extra_flags=()) -> str:
    exe = os.path.join(out_dir, "plan_probe")
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", *extra_flags, "-I", CSRC,
           os.path.join(HERE, "plan_probe.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    return build_probe(str(tmp_path_factory.mktemp("plan")))


def plan(probe, B, T, D, R, W, bf16=1) -> dict:
    out = subprocess.run([probe, str(B), str(T), str(D), str(R), str(W), str(bf16)], check=True,
                         capture_output=True, text=True).stdout
    return {k: int(v) for k, v in (line.split("=") for line in out.split())}


@pytest.mark.parametrize("R,D", [(32, 16), (16, 16), (8, 8)])
def test_fused_dz_partial_stays_inside_its_buffer_range(probe, R, D):
    # the last T whose partial [T][R] fits, and the first that does not
    t_fit = LIM // (4 * R)
    p = plan(probe, 1, t_fit, D, R, 4)
    assert p["mfma"] == 1 and p["bwd_fused_dz"] == 1
    assert t_fit * R * 4 <= LIM
    p = plan(probe, 1, t_fit + 1, D, R, 4)
    assert p["mfma"] == 1 and p["bwd_fused_dz"] == 0, "past 2 GiB of partials the separate dz pass must run"
    # the shape that used to be planned fused with a 2,147,485,696-byte partial
    p = plan(probe, 1, 2 ** 24 + 16, 16, 32, 4)
    assert p["mfma"] == 1 and p["bwd_fused_dz"] == 0


def test_fused_dz_sweep(probe):
    import numpy as np

    rng = np.random.default_rng(5)
    for _ in range(40):
        R = int(rng.choice([8, 16, 24, 32]))
        T = int(rng.integers(1, 2 ** 27))
        D = int(rng.choice([8, 16, 64]))
        W = int(rng.integers(1, 9))
        p = plan(probe, 1, T, D, R, W)
        if p["mfma"] and p["bwd_fused_dz"]:
            assert T * R * 4 <= LIM, (T, D, R, W)


def test_launches_fit_a_dispatch(probe):
    # 2^24 one-step sequences: the forward alone would need 2^24 blocks of 256 threads
    p = plan(probe, 2 ** 24, 1, 64, 32, 4)
    assert p["mfma"] == 0
    # 2^23: the fused backward's blocks of 8 waves would reach 2^32 work-items exactly
    assert plan(probe, 2 ** 23, 1, 64, 32, 4)["mfma"] == 0
    # 2^22: still the matrix cores, every grid below 2^32 work-items
    B = 2 ** 22
    p = plan(probe, B, 1, 64, 32, 4)
    assert p["mfma"] == 1 and p["bwd_fused_dz"] == 1
    fwd = p["fwd_n_cblk"] * p["fwd_n_split"] * B
    bwd = p["bwd_n_cblk"] * p["bwd_n_split"] * B
    assert fwd * 256 < 2 ** 32 and bwd * 64 * p["bwd_NW"] < 2 ** 32


def test_library_workspace_matches_plan(probe):
    lib_path = os.path.join(ROOT, "dynamic_short_convolutions_amd", "libdsc.so")
    if not os.path.exists(lib_path):
        pytest.skip("libdsc.so is not built")
    L = ctypes.CDLL(lib_path)
    L.dsc_lowrank_bwd_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int]
    L.dsc_lowrank_bwd_workspace_bytes.restype = ctypes.c_size_t
    for B, T, D, R, W in [(8, 4096, 2048, 32, 4), (1, 65536, 4096, 64, 8), (1, 2 ** 24 + 16, 16, 32, 4),
                          (3, 1000, 200, 16, 3), (2, 77, 8, 128, 8)]:
        p = plan(probe, B, T, D, R, W)
        want = p["workspace_bytes"] if p["mfma"] else 0
        assert L.dsc_lowrank_bwd_workspace_bytes(B, T, D, R, W, 1) == want, (B, T, D, R, W)
