"""The bound behind the fixed-point dQ mode (deterministic = 4), on the fp64
oracle: for query row i, every element of the unscaled dQ (dQ / softmax_scale)
and every partial sum of it over a subset of the keys (one workgroup's key
tile) is at most beta_i = |dO_i| max_j |V_j| max_jc |K_jc| in magnitude, the
maxima taken over every key row of the key/value head.  The partial sums are
what the kernel converts to int32, so a partial sum above the bound would
saturate.

Why: dQ_ic = sum_j P_ij (dP_ij - D_i) K_jc with D_i = sum_j P_ij dP_ij (the
row sum of dO_i o O_i), so |dQ_ic| <= max|K| sum_j P_ij |dP_ij - D_i|, the
mean absolute deviation of dP_ij = dO_i . V_j under the weights P_ij, which is
at most its standard deviation, at most half its range (Popoviciu's
inequality), at most |dO_i| max_j |V_j|.  The two-key case below attains it."""

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora


def beta(do, k, v, Hq):
    """[B, N, Hq] bounds from dense inputs (maxima over the whole key axis)."""
    Hkv = k.shape[2]
    a = np.sqrt(np.sum(do.astype(np.float64) ** 2, axis=-1))
    vn = np.sqrt(np.sum(v.astype(np.float64) ** 2, axis=-1)).max(axis=(0, 1))
    km = np.abs(k.astype(np.float64)).max(axis=(0, 1, 3))
    g = np.arange(Hq) // (Hq // Hkv)
    return a * (vn * km)[g]


def partial_sums(q, k, v, do, scale, causal, tile):
    """Unscaled dQ of each (row, head) split into sums over key tiles of
    `tile` keys: [B, N, Hq, n_tiles, d], from P and dS built from the oracle's
    forward (O, LSE)."""
    o, lse = ora.attention_forward(q, k, v, scale, causal)
    B, N, Hq, d = q.shape
    G = Hq // k.shape[2]
    nt = -(-N // tile)
    out = np.zeros((B, N, Hq, nt, d))
    for b in range(B):
        for h in range(Hq):
            kk, vv = k[b, :, h // G].astype(np.float64), v[b, :, h // G].astype(np.float64)
            s = q[b, :, h].astype(np.float64) @ kk.T * scale
            if causal:
                s = np.where(np.tri(N, dtype=bool), s, -np.inf)
            p = np.exp(s - lse[b, h][:, None])
            dp = do[b, :, h].astype(np.float64) @ vv.T
            dd = np.sum(do[b, :, h].astype(np.float64) * o[b, :, h], axis=-1)
            ds = p * (dp - dd[:, None])
            for t in range(nt):
                out[b, :, h, t] = ds[:, t * tile:(t + 1) * tile] @ kk[t * tile:(t + 1) * tile]
    return out


CASES = [
    # (B, N, Hq, Hkv, d, causal, q_mult): q_mult sharpens the softmax
    (1, 300, 2, 2, 64, False, 1.0),
    (2, 200, 4, 2, 64, True, 1.0),
    (1, 257, 3, 1, 128, True, 8.0),
    (1, 100, 2, 1, 32, False, 30.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_bound_holds(case):
    B, N, Hq, Hkv, d, causal, mult = case
    x = inputs.dense_inputs(B, N, Hq, Hkv, d, seed=91)
    q = x["q"] * mult
    sc = 1.0 / np.sqrt(d)
    bnd = beta(x["do"], x["k"], x["v"], Hq)
    dq = ora.attention_backward(q, x["k"], x["v"], x["do"], sc, causal)[0] / sc
    assert np.all(np.abs(dq) <= bnd[..., None] * (1 + 1e-12))
    parts = partial_sums(q, x["k"], x["v"], x["do"], sc, causal, tile=64)
    assert np.allclose(parts.sum(axis=3), dq, rtol=1e-9, atol=1e-12)
    assert np.all(np.abs(parts) <= bnd[..., None, None] * (1 + 1e-12))


def test_bound_is_attained():
    """One query (q = 0, so equal weights on two keys), V_1 = -V_2 = e_1,
    K_1 = -K_2 = e_1 and dO = e_1: dP = (1, -1), D = 0, dS = (1/2, -1/2) and
    the unscaled dQ = e_1, equal to |dO| max|V| max|K| = 1."""
    d = 4
    q = np.zeros((1, 2, 1, d))
    k = np.zeros((1, 2, 1, d))
    v = np.zeros((1, 2, 1, d))
    do = np.zeros((1, 2, 1, d))
    k[0, 0, 0, 0], k[0, 1, 0, 0] = 1.0, -1.0
    v[0, 0, 0, 0], v[0, 1, 0, 0] = 1.0, -1.0
    do[0, 1, 0, 0] = 1.0  # the second query (row 1) sees both keys
    sc = 0.5
    dq = ora.attention_backward(q, k, v, do, sc, False)[0] / sc
    bnd = beta(do, k, v, 1)
    assert abs(dq[0, 1, 0, 0] - 1.0) < 1e-12
    assert abs(bnd[0, 1, 0] - 1.0) < 1e-12
    assert np.allclose(dq[0, 1, 0, 1:], 0.0)
