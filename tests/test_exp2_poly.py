"""Host-side pins of the forward's software exponential (poly_exp2).

2^x = 2^n * p(x - n) with n = round(x) and p a cubic fitted to 2^f on
[-1/2, 1/2] ([FA4N] co-design list: exponentials emulated on the FMA units).
The device function is compiled for the host (hipcc) and checked against 2^x
in float64: relative error within the cubic's minimax error (8.4e-5) plus a
few fp32 roundings over the whole range the forward feeds it (scores minus a
reference maximum, at most the rescale threshold 8 above it), exact zero for a
masked score (-inf) and for arguments below the fp32 range, exact powers of
two at integers; and the constants in the header are the ones the fit script
derives."""

import os
import re
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
FIT_ERR = 8.4e-5          # largest relative error of the fp32 cubic on [-1/2, 1/2]
ROUNDING = 6 * 2.0 ** -24  # fp32 roundings of f = x - n and of the Horner steps


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("exp2") / "exp2_check")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17",
                    os.path.join(HERE, "host", "exp2_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def poly(exe, x):
    x = np.asarray(x, dtype=np.float32)
    text = "\n".join(f"{b:08x}" for b in x.view(np.uint32)) + "\n"
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return np.array([int(t, 16) for t in out.split()], dtype=np.uint32).view(np.float32)


def test_relative_error_over_the_forward_range(checker):
    rng = np.random.Generator(np.random.PCG64(5))
    x = np.concatenate([np.linspace(-126.0, 8.5, 200001, dtype=np.float32),
                        rng.uniform(-30.0, 8.5, 100000).astype(np.float32),
                        # both sides of every rounding boundary n + 1/2
                        np.nextafter(np.arange(-40.5, 9.0, 1.0, dtype=np.float32), np.float32(-1e9)),
                        np.nextafter(np.arange(-40.5, 9.0, 1.0, dtype=np.float32), np.float32(1e9))])
    y = poly(checker, x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y / ref - 1.0)
    assert np.max(rel) <= FIT_ERR + ROUNDING, float(np.max(rel))
    # the error is that of the fit, not much smaller: the cubic is in use
    assert np.max(rel) > 0.5 * FIT_ERR


def test_special_arguments(checker):
    x = np.array([-np.inf, -1000.0, -160.0, -151.0, 0.0, 1.0, -1.0, 8.0, -126.0], dtype=np.float32)
    y = poly(checker, x)
    assert y[0] == 0.0 and y[1] == 0.0 and y[2] == 0.0 and y[3] == 0.0   # masked, underflow
    # integers: 2^n * p(0), p(0) = the constant coefficient
    c0 = np.float32(9.999195933e-01)
    for xi, yi in zip(x[4:], y[4:]):
        assert yi == np.float32(np.ldexp(c0, int(xi))), (xi, yi)
    # denormal results keep an absolute error below the smallest denormal's size
    xd = np.linspace(-149.0, -126.0, 2001, dtype=np.float32)
    yd = poly(checker, xd).astype(np.float64)
    assert np.max(np.abs(yd - np.exp2(xd.astype(np.float64)))) <= 2.0 ** -149 + 2.0 ** -126 * FIT_ERR


def test_header_constants_come_from_the_fit():
    from exact_attention_80_amd import exp2_fit
    coeffs, err = exp2_fit.fit()
    text = open(os.path.join(ROOT, "exact_attention_80_amd", "csrc", "fa_exp2.h")).read()
    header = [float(re.search(rf"kExp2C{k} = ([0-9.e+-]+)f", text).group(1)) for k in range(4)]
    assert np.allclose(np.float32(header), coeffs, rtol=2.0 ** -22, atol=0.0), (header, coeffs)
    assert err <= FIT_ERR
