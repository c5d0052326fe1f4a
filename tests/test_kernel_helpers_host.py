"""The library's device-side bf16 rounding helpers, compiled for the host and
checked on the CPU: fp64 -> bf16 against the oracle's pinned rounding and the
hand-derived golden cases, fp32 -> bf16 against torch."""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = tmp_path_factory.mktemp("hostcheck") / "round_check"
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "kv_cached_decode_amd", "csrc"),
                    os.path.join(HERE, "host_round_check.cpp"), "-o", str(exe)], check=True)
    return str(exe)


def run(exe, xs):
    inp = "\n".join(float(x).hex() for x in xs) + "\n"
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    a = np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()], np.uint32)
    return a[:, 0].astype(np.uint16), a[:, 1].astype(np.uint16)


def test_f64_rounding_matches_oracle(driver):
    rng = np.random.default_rng(5)
    xs = np.concatenate([
        rng.standard_normal(20000) * 3.0,
        rng.standard_normal(3000) * 1e-39,
        rng.standard_normal(3000) * 1e37,
        # values exactly at and next to bf16 ties, below fp32 precision too
        (rng.integers(128, 256, 3000) * 2 + 1) * 2.0 ** -9 * (1 + rng.choice([-1, 0, 1], 3000) * 2.0 ** -40),
        [0.0, -0.0, float("inf"), float("-inf")] + [float.fromhex(h) for h in ("0x1.fep127", "0x1.ffp127", "0x1p-133", "0x1p-134")],
    ])
    got, _ = run(driver, xs)
    want = np.array([oracle.bf16_from_double(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, want), f"{int((got != want).sum())} of {xs.size} differ"


def test_f64_rounding_golden(driver):
    with open(os.path.join(HERE, "golden", "bf16_rounding_cases.json")) as f:
        cases = json.load(f)["cases"]
    xs = [float(c["x"]) if "inf" in c["x"] else float.fromhex(c["x"]) for c in cases]
    got, _ = run(driver, xs)
    for g, c in zip(got, cases):
        assert int(g) == int(c["bits"], 16), c


def test_f32_rounding_matches_torch(driver):
    rng = np.random.default_rng(6)
    xs = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                         ((rng.integers(128, 256, 2000) * 2 + 1) * 2.0 ** -9).astype(np.float32),
                         np.float32([3.39e38, -3.39e38, 1e-40, 0.0])])
    _, got = run(driver, xs.astype(np.float64))
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
