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
