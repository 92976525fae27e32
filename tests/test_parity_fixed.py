"""GPU parity of the fixed-point dQ mode (deterministic = 4): every dQ
contribution of row i is rounded to a multiple of 2^-e_i and added as an
int32, where e_i comes from the bound beta_i = |dO_i| max_j |V_j| max |K| of
the row's unscaled dQ (the K/V maxima over every key row of the key/value
head).  The adds are exact, so the result is the same bit for bit in any
order of the workgroups.

The checks, besides the oracle bars of the other modes:
  * dK and dV do not depend on the dQ reduction: bit-identical to the fp32
    atomic mode (0), which walks the query tiles in the same order (the
    ordered mode 1 walks a causal key tile's query tiles the other way);
  * dQ against mode 1 element by element, within a bound derived from the
    two reductions: the fixed-point rounding (half a step 2^-e_i per add,
    at most n_kt adds, plus the int32 -> fp32 conversion of a sum below
    2^30 steps), the fp32 summation error of mode 1 (n_kt 2^-24 beta_i, since
    the partial sums' magnitudes add up to at most beta_i), and the two bf16
    roundings of the outputs.  e_i is recomputed here from the inputs;
  * bit-identical results over repeated runs and with the tile order of the
    scheduler switched off;
  * a row whose bound is not finite (an infinite dO element) comes out NaN
    while every other row keeps its value."""

import math

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora

from gpu_helpers import TOL_GRAD, rel_fro, say, scale_for, to_dev, to_host

pytestmark = pytest.mark.gpu

FIXED = 4
ORDERED = 1


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa as _fa
    return _fa


def same(a, b) -> bool:
    import torch
    return a.shape == b.shape and bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))


def row_bound(do, k, v):
    """beta = |dO_row| max_j |V_j| max |K| per (token, query head), from the
    inputs in fp64; do: [T, Hq, d], k, v: [Tk, Hkv, d]."""
    Hq, Hkv = do.shape[1], k.shape[1]
    a = np.sqrt(np.sum(do.astype(np.float64) ** 2, axis=-1))             # [T, Hq]
    vn = np.sqrt(np.sum(v.astype(np.float64) ** 2, axis=-1)).max(axis=0)  # [Hkv]
    km = np.abs(k.astype(np.float64)).max(axis=(0, 2))                    # [Hkv]
    g = np.arange(Hq) // (Hq // Hkv)
    return a * (vn * km)[g][None, :]


def dq_tolerance(beta, ref_a, ref_b, scale, n_kt):
    """Per-element bound on |dQ_fixed - dQ_ordered| (module docstring)."""
    # the step 2^-e_i = 2^(k - 29) for beta < 2^k; taken one power of two up, since
    # the kernel's fp32 beta may cross a power of two that this fp64 one does not
    _, k = np.frexp(beta)
    step = np.ldexp(1.0, k - 28)
    delta = scale * (n_kt * step / 2 + 32 * step + n_kt * 2.0 ** -24 * beta)
    mag = np.maximum(np.abs(ref_a), np.abs(ref_b))
    return 2.0 ** -7 * mag + 1.01 * delta[..., None] + 1e-30


def check_fixed(dq4, dq1, do, k, v, scale, n_keys):
    a, b = to_host(dq4), to_host(dq1)
    beta = row_bound(do.reshape(-1, *do.shape[-2:]), k.reshape(-1, *k.shape[-2:]),
                     v.reshape(-1, *v.shape[-2:])).reshape(a.shape[:-1])
    tol = dq_tolerance(beta, a, b, scale, math.ceil(n_keys / 128) + 1)
    excess = float(np.max(np.abs(a - b) / tol)) if a.size else 0.0
    say(f"dQ fixed vs ordered: worst |diff| / bound = {excess:.3g}")
    assert excess <= 1.0


DENSE = [
    (1, 128, 2, 2, 64),
    (1, 200, 2, 2, 64),
    (2, 333, 4, 4, 128),
    (1, 1, 2, 1, 128),
    (2, 300, 8, 2, 128),
    (1, 260, 4, 1, 64),
    (1, 1024, 4, 2, 128),
    (2, 250, 3, 1, 64),
    (1, 300, 2, 2, 256),
    (2, 129, 4, 2, 256),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", DENSE, ids=lambda s: "x".join(map(str, s)))
def test_dense(fa, shape, causal):
    B, N, Hq, Hkv, d = shape
    say(f"fixed dense B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    x = inputs.dense_inputs(B, N, Hq, Hkv, d, seed=81)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    sc = scale_for(d)
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=causal, softmax_scale=sc)
    g4 = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal, softmax_scale=sc,
                deterministic=FIXED)
    g1 = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal, softmax_scale=sc,
                deterministic=ORDERED)
    g0 = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal, softmax_scale=sc,
                deterministic=0)
    assert same(g4[1], g0[1]) and same(g4[2], g0[2])
    check_fixed(g4[0], g1[0], x["do"], x["k"], x["v"], sc, N)
    rg = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], sc, causal)
    errs = {n: rel_fro(to_host(a), r) for n, a, r in zip(("dq", "dk", "dv"), g4, rg)}
    say(f"errors {errs}")
    assert max(errs.values()) <= TOL_GRAD


VARLEN = [
    ([1, 5, 130, 257, 64, 600, 33], 4, 2, 128),
    ([300, 1, 1000, 129], 2, 2, 64),
    ([513, 40], 2, 1, 256),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"n{len(c[0])}h{c[1]}{c[2]}d{c[3]}")
def test_varlen(fa, case, causal):
    import torch
    lengths, Hq, Hkv, d = case
    say(f"fixed varlen lengths={lengths} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    x = inputs.varlen_inputs(lengths, Hq, Hkv, d, seed=82)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    cu = torch.from_numpy(x["cu_seqlens"]).to("cuda")
    sc = scale_for(d)
    o, lse = fa.varlen_fwd(t["q"], t["k"], t["v"], cu, causal=causal, softmax_scale=sc)
    g4 = fa.varlen_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cu, causal=causal,
                       softmax_scale=sc, deterministic=FIXED)
    g1 = fa.varlen_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cu, causal=causal,
                       softmax_scale=sc, deterministic=ORDERED)
    g0 = fa.varlen_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cu, causal=causal,
                       softmax_scale=sc, deterministic=0)
    assert same(g4[1], g0[1]) and same(g4[2], g0[2])
    check_fixed(g4[0], g1[0], x["do"], x["k"], x["v"], sc, max(lengths))
    rg = ora.varlen_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens"], sc, causal)
    errs = {n: rel_fro(to_host(a), r) for n, a, r in zip(("dq", "dk", "dv"), g4, rg)}
    say(f"errors {errs}")
    assert max(errs.values()) <= TOL_GRAD


QK = [
    ([1, 17, 0, 300, 1], [900, 2049, 40, 700, 500], 8, 2, 128),
    ([1, 300, 0, 65, 7], [700, 300, 40, 129, 1], 4, 2, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", QK, ids=lambda c: f"n{len(c[0])}h{c[2]}{c[3]}d{c[4]}")
def test_separate_lengths(fa, case, causal):
    import torch
    lq, lk, Hq, Hkv, d = case
    say(f"fixed varlen_qk lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    x = inputs.varlen_qk_inputs(lq, lk, Hq, Hkv, d, seed=83)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    cq = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    ck = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    sc = scale_for(d)
    o, lse = fa.varlen_qk_fwd(t["q"], t["k"], t["v"], cq, ck, causal=causal, softmax_scale=sc)
    g4 = fa.varlen_qk_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=causal,
                          softmax_scale=sc, deterministic=FIXED)
    g1 = fa.varlen_qk_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=causal,
                          softmax_scale=sc, deterministic=ORDERED)
    g0 = fa.varlen_qk_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=causal,
                          softmax_scale=sc, deterministic=0)
    assert same(g4[1], g0[1]) and same(g4[2], g0[2])
    check_fixed(g4[0], g1[0], x["do"], x["k"], x["v"], sc, max(lk))
    rg = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                                x["cu_seqlens_k"], sc, causal)
    errs = {n: rel_fro(to_host(a), r) for n, a, r in zip(("dq", "dk", "dv"), g4, rg)}
    say(f"errors {errs}")
    assert max(errs.values()) <= TOL_GRAD


def test_bit_identical_in_any_order(fa, monkeypatch):
    """Repeated runs, and the tile order of the dense and packed backward with
    the longest-first order and the XCD grouping switched off: the same bits."""
    import torch
    say("fixed bit identity dense B=2 N=1100 Hq=8 Hkv=2 d=128 causal, packed batch")
    x = inputs.dense_inputs(2, 1100, 8, 2, 128, seed=84)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=True)
    lengths = [700, 3, 128, 1029, 64]
    xv = inputs.varlen_inputs(lengths, 4, 1, 128, seed=85)
    tv = {n: to_dev(xv[n]) for n in ("q", "k", "v", "do")}
    cu = torch.from_numpy(xv["cu_seqlens"]).to("cuda")
    ov, lsev = fa.varlen_fwd(tv["q"], tv["k"], tv["v"], cu, causal=True)

    def run():
        g = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=True, deterministic=FIXED)
        gv = fa.varlen_bwd(tv["q"], tv["k"], tv["v"], ov, lsev, tv["do"], cu, causal=True,
                           deterministic=FIXED)
        torch.cuda.synchronize()
        return tuple(a.clone() for a in g + gv)

    ref = run()
    for rep in range(4):
        if rep == 2:
            monkeypatch.setenv("FA_SCHED", "natural")
        for a, b in zip(run(), ref):
            assert same(a, b), rep


def test_non_finite_bound_gives_nan_rows(fa):
    import torch
    B, N, Hq, Hkv, d = 1, 300, 4, 2, 128
    say(f"fixed non-finite dO row B={B} N={N} Hq={Hq} Hkv={Hkv} d={d}")
    x = inputs.dense_inputs(B, N, Hq, Hkv, d, seed=86)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=True)
    do = t["do"].clone()
    do[0, 250, 1, 7] = float("inf")
    dq4 = fa.bwd(t["q"], t["k"], t["v"], o, lse, do, causal=True, deterministic=FIXED)[0]
    dq1 = fa.bwd(t["q"], t["k"], t["v"], o, lse, do, causal=True, deterministic=ORDERED)[0]
    torch.cuda.synchronize()
    bad = torch.zeros(B, N, Hq, dtype=torch.bool, device="cuda")
    bad[0, 250, 1] = True
    assert bool(torch.isnan(dq4[bad]).all())
    # every other row depends only on finite values and keeps its value
    assert bool(torch.isfinite(dq4[~bad]).all())
    xd = x["do"].copy()
    xd[0, 250, 1, 7] = np.inf
    beta = row_bound(xd[0], x["k"][0], x["v"][0])[None]
    a, b = to_host(dq4), to_host(dq1)
    keep = ~bad.cpu().numpy()
    tol = dq_tolerance(beta, a, b, scale_for(d), math.ceil(N / 128) + 1)
    assert float(np.max((np.abs(a - b) / tol)[keep])) <= 1.0
