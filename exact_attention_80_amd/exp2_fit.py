"""Coefficients of the cubic that the forward's software exponential uses.

The forward can compute part of its exponentials without the hardware
exponential instruction ([FA4N] co-design list: an exponential emulated by a
polynomial on the FMA units; [FA4B] 5.3): 2^x = 2^n * 2^f with n = round(x)
and f = x - n in [-1/2, 1/2] (Cody-Waite range reduction with the exact
power-of-two step), and 2^f from a cubic.  The cubic here minimises the
largest relative error of p(f) / 2^f - 1 on [-1/2, 1/2] (Lawson's iteratively
reweighted least squares on a dense grid, which converges to the minimax fit),
rounded to fp32.  A probability is rounded to bf16 (8 significant bits) right
after, so a relative error near 1e-4 is far below that rounding.

    python -m exact_attention_80_amd.exp2_fit     # prints the coefficients

The printed values are the kExp2C* constants in csrc/fa_common.h.
"""

from __future__ import annotations

import numpy as np

DEGREE = 3
GRID = 20001
ITERATIONS = 200


def fit(degree: int = DEGREE, grid: int = GRID, iterations: int = ITERATIONS):
    """Minimax-relative-error polynomial coefficients (constant term first)
    of 2^f on [-1/2, 1/2], as float32, and the fit's largest relative error."""
    f = np.linspace(-0.5, 0.5, grid)
    y = np.exp2(f)
    vander = np.vander(f, degree + 1, increasing=True)
    w = np.full(grid, 1.0 / grid)
    for _ in range(iterations):
        a = vander * (w / y)[:, None]
        c, *_ = np.linalg.lstsq(a, w, rcond=None)
        err = np.abs(vander @ c / y - 1.0)
        w = w * err
        w /= w.sum()
    c32 = c.astype(np.float32)
    return c32, float(np.max(np.abs(vander @ c32.astype(np.float64) / y - 1.0)))


if __name__ == "__main__":
    coeffs, err = fit()
    for k, v in enumerate(coeffs):
        print(f"kExp2C{k} = {float(v):.9e}f  ({v.view(np.uint32):#010x})")
    print(f"max relative error of the fp32 coefficients on [-1/2, 1/2]: {err:.3e}")
