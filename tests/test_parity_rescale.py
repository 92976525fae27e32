"""GPU parity on inputs that drive the forward's conditional rescale.

The forward keeps a stale reference maximum per row and rescales its
accumulator only when a row maximum grows by more than a threshold (8 in log2
units), so probabilities stay below 2^8 and the row sum below N 2^8 ([FA4N]
co-design list: conditional softmax rescaling; [FA2] "Core method" 1: the
online softmax and its logsumexp).  With N(0, 1) inputs and scale 1/sqrt(d) a
row maximum practically never grows by that much after the first 64-key tile,
so these inputs are built to make it grow:

  * ramp: key j is scaled by 1 + 8 j / N, so the maxima of causal and
    non-causal rows rise by tens of log2 units along the keys and every wave
    rescales several times;
  * plateau: the first 64 keys score about M and every later key about
    M + 7.93 (log2 units), just under the threshold: the reference maximum
    never moves after the first tile and the row sum reaches about 0.9 N 2^8,
    close to the largest it can be; its companion at M + 8.13 rescales at the
    second tile.

Each case first checks on the CPU, from the oracle's scores, that the inputs
do what they are for; then it compares the forward and backward with the
oracle (the acceptance bars), and the default build with a build whose
threshold is 0 (a rescale at every growth of a row maximum): the result is
mathematically independent of the threshold, so the LSE must agree within the
fp32 rounding of the row sum and O within the bf16 rounding of the
probabilities (the two builds round different multiples of them).
"""

import math

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora

from gpu_helpers import (TOL_GRAD, TOL_LSE, max_abs, o_excess, rel_fro, say, scale_for, to_dev,
                         to_host)

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)
TAU = 8.0          # the default build's threshold (log2 units)
KEY_TILE = 64      # keys per forward key tile


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa as _fa
    return _fa


@pytest.fixture(scope="module")
def fa_tau0(fa):
    return fa.load_variant("tau0")


def head_views(x, G, b, h):
    g = h // G
    return x["q"][b, :, h], x["k"][b, :, g], x["v"][b, :, g], x["do"][b, :, h]


def tile_growth(qh, kh, scale, causal):
    """Per query row: the largest amount (log2 units) by which the maximum of
    a later 64-key tile exceeds the maximum of the row's first tile; -inf for
    rows that see a single tile."""
    s = ora.head_scores(qh, kh, scale, causal) * LOG2E
    n = kh.shape[0]
    first = s[:, :KEY_TILE].max(axis=1)
    grow = np.full(s.shape[0], -np.inf)
    for j0 in range(KEY_TILE, n, KEY_TILE):
        m = s[:, j0:j0 + KEY_TILE].max(axis=1)
        grow = np.maximum(grow, m - first)
    return grow


def oracle_all(x, scale, causal):
    ro, rlse = ora.attention_forward(x["q"], x["k"], x["v"], scale, causal)
    pv, _ = ora.attention_forward(x["q"], x["k"], np.abs(x["v"]), scale, causal)
    rdq, rdk, rdv = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    return ro, rlse, pv, (rdq, rdk, rdv)


def run_and_compare(fa, fa_tau0, x, scale, causal, check_dq=True):
    """Forward and backward against the oracle; the threshold-0 build against
    the default one.  check_dq=False leaves out dQ where it is ill-conditioned
    (see the plateau tests)."""
    import torch
    B, N, Hq, d = x["q"].shape
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=causal, softmax_scale=scale)
    grads = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal, softmax_scale=scale)
    o0, lse0 = fa.fwd(t["q"], t["k"], t["v"], causal=causal, softmax_scale=scale, lib=fa_tau0)
    torch.cuda.synchronize()
    ro, rlse, pv, rgrads = oracle_all(x, scale, causal)
    o_h, lse_h, o0_h, lse0_h = (to_host(a) for a in (o, lse, o0, lse0))
    errs = dict(o_excess=o_excess(o_h, ro, pv, N), lse=max_abs(lse_h, rlse))
    for name, g, r in zip(("dq", "dk", "dv"), grads, rgrads):
        errs[name] = rel_fro(to_host(g), r)
    # threshold 0 against threshold 8: LSE within (N + 16) 2^-24 (both row sums
    # are fp32 sums of at most N unrounded probabilities) plus 2^-18 (|LSE| + 1)
    # for the fp32 sum m + log2 l; O within one bf16 ulp of O* (each build
    # rounds once) plus twice 2^-8 + (N + 64) 2^-24 of sum_j P_ij |V_jd|
    lse_bound = (N + 16) * 2.0 ** -24 + 2.0 ** -18 * (np.abs(rlse) + 1.0)
    a = np.abs(ro)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-30))) - 7)
    o_bound = np.where(a > 0, ulp, 2.0 ** -133) + 2.0 * (2.0 ** -8 + (N + 64) * 2.0 ** -24) * pv
    errs["tau0_lse"] = float(np.max(np.abs(lse_h - lse0_h) / lse_bound))
    errs["tau0_o"] = float(np.max(np.abs(o_h - o0_h) / np.maximum(o_bound, 1e-30)))
    say(f"errors {errs}")
    assert errs["o_excess"] <= 1.0 and errs["lse"] <= TOL_LSE
    assert (errs["dq"] <= TOL_GRAD or not check_dq) and errs["dk"] <= TOL_GRAD
    assert errs["dv"] <= TOL_GRAD
    assert errs["tau0_lse"] <= 1.0 and errs["tau0_o"] <= 1.0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_ramp_rescales_several_times(fa, fa_tau0, d, causal):
    B, N, Hq, Hkv = 1, 700, 4, 2
    say(f"ramp B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    x = inputs.ramp_inputs(B, N, Hq, Hkv, d, seed=31)
    sc = scale_for(d)
    # the inputs rescale: in every head most rows' maxima grow by more than
    # the threshold after the first tile, some by several thresholds
    for h in range(Hq):
        g = tile_growth(*head_views(x, Hq // Hkv, 0, h)[:2], sc, causal)
        assert np.mean(g > TAU) > 0.5 and np.max(g) > 2 * TAU, (h, np.mean(g > TAU), np.max(g))
    run_and_compare(fa, fa_tau0, x, sc, causal)


def plateau_level(d, scale, lo, hi):
    """A bf16 key level whose score against an all-ones query lies between lo
    and hi log2 units (the bf16 grid there is about 0.03 to 0.05 units wide)."""
    t = np.float32((lo + hi) / 2 / (LOG2E * scale * d))
    u = int(np.asarray(inputs.bf16_bits(inputs.bf16_round(t))).reshape(-1)[0])
    for step in range(64):
        for cand in (u - step, u + step):
            level = float(inputs.bits_to_f32(np.array([cand], dtype=np.uint16))[0])
            if lo <= LOG2E * scale * d * level <= hi:
                return level
    raise ValueError("no bf16 level in range")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_plateau_just_below_threshold(fa, fa_tau0, d, causal):
    """Row sums up to about 0.9 N 2^8 without any rescale after the first tile.

    dQ is not compared here: with every later key equal, dQ_i = scale
    sum_j dS_ij k_j nearly cancels (the dS_ij of a row sum to zero), while
    rounding each dS_ij to bf16 leaves errors of 2^-8 |dS_ij| |k_j| that do not
    cancel, far above 2e-2 of the tiny exact dQ (the ramp cases check dQ)."""
    N, Hq, Hkv = 2000, 2, 1
    sc = scale_for(d)
    level = plateau_level(d, sc, 7.90, 7.96)
    say(f"plateau N={N} Hq={Hq} d={d} causal={causal} level={level}")
    x = inputs.plateau_inputs(N, Hq, Hkv, d, level, seed=32)
    for h in range(Hq):
        qh, kh = head_views(x, Hq, 0, h)[:2]
        g = tile_growth(qh, kh, sc, causal)
        live = g > -np.inf
        # every later tile stays under the threshold, within 0.25 of it
        assert np.all(g[live] < TAU) and np.all(g[live] > TAU - 0.25), (g[live].min(), g[live].max())
        # the row sum in the reference of the first tile: close to N 2^8
        s = ora.head_scores(qh, kh, sc, causal) * LOG2E
        ref = s[:, :KEY_TILE].max(axis=1)
        lsum = np.exp2(s - ref[:, None]).sum(axis=1)
        assert lsum[-1] > 0.85 * N * 2 ** TAU, lsum[-1]
    run_and_compare(fa, fa_tau0, x, sc, causal, check_dq=False)


@pytest.mark.parametrize("causal", [False, True])
def test_plateau_just_above_threshold(fa, fa_tau0, causal):
    """The same plateau 0.1 above the threshold: every row rescales once, at
    its second tile (dQ left out as above)."""
    N, Hq, Hkv, d = 2000, 2, 1, 128
    sc = scale_for(d)
    level = plateau_level(d, sc, 8.10, 8.16)
    say(f"plateau above N={N} d={d} causal={causal} level={level}")
    x = inputs.plateau_inputs(N, Hq, Hkv, d, level, seed=33)
    for h in range(Hq):
        g = tile_growth(*head_views(x, Hq, 0, h)[:2], sc, causal)
        live = g > -np.inf
        assert np.all(g[live] > TAU) and np.all(g[live] < TAU + 0.3), (g[live].min(), g[live].max())
    run_and_compare(fa, fa_tau0, x, sc, causal, check_dq=False)
