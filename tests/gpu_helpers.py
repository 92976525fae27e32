"""Helpers shared by the GPU tests: upload seeded inputs, compare with the oracle."""

from __future__ import annotations

import math

import numpy as np

from exact_attention_80_amd import inputs

# Acceptance tolerances for bf16 inputs (oracle evaluated on the same bf16 values):
# O max abs error, LSE max abs error, relative Frobenius error of dQ, dK, dV.
TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_GRAD = 2e-2


def o_tolerance(ref: np.ndarray) -> np.ndarray:
    """Per-element bound on |O - O*|: TOL_O wherever |O*| < 4.  From |O*| = 4 up,
    the bf16 grid of the stored output is coarser than TOL_O (half an ulp is
    2^-6 at 4), so the bound there is half a bf16 ulp of O* plus 2^-8 |O*|, the
    worst case of rounding every probability to bf16 (relative 2^-9) before the
    P V product."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    return np.where(a >= 4.0, np.maximum(TOL_O, 2.0 ** (e - 8) + a * 2.0 ** -8), TOL_O)


def o_excess(o: np.ndarray, ref: np.ndarray) -> float:
    """Largest |O - O*| / bound (<= 1 passes)."""
    return float(np.max(np.abs(o - ref) / o_tolerance(ref))) if o.size else 0.0


def to_dev(x: np.ndarray):
    import torch
    bits = inputs.bf16_bits(x).view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(bits)).to("cuda").view(torch.bfloat16)


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_fro(a, b) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (nb if nb > 0 else 1.0)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def scale_for(d: int) -> float:
    return 1.0 / math.sqrt(d)


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
