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


def o_tolerance(ref: np.ndarray, pv_abs, n_keys: int) -> np.ndarray:
    """Per-element bound on |O - O*|: the acceptance bar TOL_O, or where the
    forward's own arithmetic can be further off in the worst case, that worst
    case:
      half a bf16 ulp of O*                  (the final rounding of O)
      + 2^-8 sum_j P_ij |V_jd|               (every probability is rounded to
                                              bf16, relative error <= 2^-8, before
                                              the P V product, while the row sum
                                              is taken from the unrounded values)
      + (n_keys + 64) 2^-24 sum_j P_ij |V_jd| (the fp32 sums of the row sum and of
                                              P V over at most n_keys keys)
    From |O*| = 4 up the first term alone (2^-6) exceeds TOL_O; below, the
    worst case exceeds it only where the probabilities are concentrated on a
    few large values of V (sum_j P_ij |V_jd| of several units), since the
    rounding errors of many small probabilities cancel.
    pv_abs is sum_j P_ij |V_jd| (the oracle's forward with |V| as the values),
    or any upper bound of it, such as max_j |V_jd| (the P_ij sum to one)."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    pv = np.broadcast_to(np.asarray(pv_abs, dtype=np.float64), a.shape)
    derived = 2.0 ** (e - 8) + (2.0 ** -8 + (n_keys + 64) * 2.0 ** -24) * pv
    return np.maximum(TOL_O, derived)


def o_excess(o: np.ndarray, ref: np.ndarray, pv_abs, n_keys: int, extra=0.0) -> float:
    """Largest |O - O*| / bound (<= 1 passes); see o_tolerance.  `extra` is
    added to the bound (the fp8 forwards' score error, see its tests)."""
    if not o.size:
        return 0.0
    return float(np.max(np.abs(o - ref) / (o_tolerance(ref, pv_abs, n_keys) + extra)))


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
