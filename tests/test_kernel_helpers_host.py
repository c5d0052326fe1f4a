"""The library's device-side bf16 rounding helpers, compiled for the host and
checked on the CPU: fp64 -> bf16 against the oracle's pinned rounding and the
hand-derived golden cases, fp32 -> bf16 against torch."""
import json
import math
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


# --- rotary sine and cosine (csrc/rope_math.h) ---------------------------------

def _pi_decimal(digits=70):
    """pi from Machin's formula, pi = 16 atan(1/5) - 4 atan(1/239)."""
    from decimal import Decimal, getcontext
    getcontext().prec = digits + 10

    def atan_inv(n):
        x = Decimal(1) / n
        x2, t, s, k = x * x, x, Decimal(0), 0
        while True:
            term = t / (2 * k + 1)
            if abs(term) < Decimal(10) ** -(digits + 5):
                return s
            s += term if k % 2 == 0 else -term
            t *= x2
            k += 1
    return 16 * atan_inv(5) - 4 * atan_inv(239)


def _exact_sincos(x, pi):
    """sin x, cos x of a double to ~60 digits: exact reduction by pi/2 in
    decimal arithmetic, then the Taylor series."""
    from decimal import Decimal
    d = Decimal(x)                      # exact value of the double
    h = pi / 2
    k = int((d / h).to_integral_value())
    r = d - k * h
    s, c, term, n = Decimal(0), Decimal(0), Decimal(1), 0
    while True:                         # term = r^n / n!
        if n % 4 == 0:
            c += term
        elif n % 4 == 1:
            s += term
        elif n % 4 == 2:
            c -= term
        else:
            s -= term
        n += 1
        term = term * r / n
        if abs(term) < Decimal(10) ** -65:
            break
    s, c = {0: (s, c), 1: (c, -s), 2: (-s, -c), 3: (-c, s)}[k % 4]
    return float(s), float(c), s, c


@pytest.fixture(scope="module")
def sincos_driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = tmp_path_factory.mktemp("sincos") / "sincos_check"
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "kv_cached_decode_amd", "csrc"),
                    os.path.join(HERE, "host_sincos_check.cpp"), "-o", str(exe)], check=True)
    return str(exe)


def test_rotary_sincos_within_two_ulps(sincos_driver):
    """The kernels' fp64 sine and cosine of pos * theta_i (both RoPE paths use
    it) against a 60-digit reference: rotary angles of two bases, points next
    to multiples of pi/2 and pi/4 (reduction and quadrant edges), random
    angles up to the fast path's limit and a few past it."""
    from decimal import Decimal
    rng = np.random.default_rng(11)
    xs = []
    for base in (10000.0, 500000.0):
        theta = base ** (-np.arange(64) * 2.0 / 128)
        pos = np.concatenate([np.arange(0, 40), rng.integers(0, 1 << 20, 40)])
        xs += list((pos[:, None].astype(np.float64) * theta[None, :]).ravel()[::7])
    for k in list(range(1, 40)) + list(rng.integers(40, 1 << 20, 60)):
        for frac in (0.5, 0.25, 0.75):
            v = float(k) * (np.pi * frac)
            xs += [v, np.nextafter(v, 0.0), np.nextafter(v, 1e9)]
    xs += list(rng.uniform(0.0, 1.6e6, 600)) + [1.6e6, 3.2e6, 1e9, 0.0, 1e-300, 2.0 ** -30]
    inp = "\n".join(float(x).hex() for x in xs) + "\n"
    out = subprocess.run([sincos_driver], input=inp, capture_output=True, text=True, check=True).stdout
    got = np.array([[float.fromhex(t) for t in line.split()] for line in out.strip().splitlines()])
    pi = _pi_decimal()
    worst = 0.0
    for x, (gs, gc) in zip(xs, got):
        _, _, es, ec = _exact_sincos(float(x), pi)
        for g, e in ((gs, es), (gc, ec)):
            ulp = math.ulp(float(e)) if float(e) != 0.0 else 2.0 ** -1074
            err = float(abs(Decimal(g) - e)) / ulp
            # values near zero (angle near a multiple of pi/2): the error is
            # bounded by the reduction's absolute error, not relative
            err = min(err, float(abs(Decimal(g) - e)) / 2.0 ** -60)
            worst = max(worst, err)
            assert err <= 2.0, (float(x).hex(), g, float(e), err)
    print(f"rotary sincos: worst {worst:.2f} ulp over {len(xs)} angles")
