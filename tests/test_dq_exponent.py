"""Host-side check of the fixed-point dQ exponent (deterministic = 4).

A row whose dQ bound is beta accumulates multiples of 2^-e in int32.  The
device function is compiled for the host here (hipcc) and checked against
its definition, with exact rational arithmetic: for finite beta > 0,
beta 2^e < 2^29 (every contribution and every sum of them stays below 2^29
steps, two bits short of int32's limit) and beta 2^e >= 2^28 (no coarser
than it must be); beta = 0 gives 29; +inf and NaN give the non-finite
marker 2^20.  The cases cover powers of two exactly, their neighbours,
subnormals and the largest finite float."""

import os
import shutil
import struct
import subprocess
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
MARKER = 1 << 20


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("dq_exponent") / "dq_exponent_check")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17",
                    os.path.join(HERE, "host", "dq_exponent_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def exponents(exe, values):
    text = "".join(f"{bits(v):08x}\n" for v in values)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return [int(x) for x in out.split()]


def test_exponent_matches_definition(checker):
    f32 = np.float32
    vals = [0.0, 1.0, 0.5, 2.0, 3.0, 1000.0, 1e-30, 1e30, 2.0 ** -149, 2.0 ** -126,
            float(np.finfo(np.float32).max)]
    for p in range(-140, 127, 7):
        x = f32(2.0) ** p
        vals += [float(x), float(np.nextafter(x, f32(0))), float(np.nextafter(x, f32(np.inf)))]
    g = np.random.Generator(np.random.PCG64(7))
    vals += [float(f32(v)) for v in np.exp(g.uniform(-80, 80, 200))]
    got = exponents(checker, vals)
    for v, e in zip(vals, got):
        if v == 0.0:
            assert e == 29
            continue
        scaled = Fraction(v) * (Fraction(2) ** e)
        assert scaled < 2 ** 29, (v, e)
        assert scaled >= 2 ** 28, (v, e)


def test_non_finite_bound_is_marked(checker):
    assert exponents(checker, [float("inf"), float("nan")]) == [MARKER, MARKER]
