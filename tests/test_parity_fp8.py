"""GPU parity of the fp8-score forwards (dense, and packed with separate query
and key lengths): Q and K arrive as OCP e4m3 bytes with per-tensor descale
factors, V as bf16.  The oracle runs the fp64 forward on
the values the bytes stand for (descale * decoded value), so the only
differences left are the kernel's accumulation and its bf16 P and O, as for
the bf16 forward, and the same tolerances apply at the scale of these inputs.

The fp8 matrix instruction does not round its 64-term sum like a chain of fp32
additions: on the same operand values its score error was measured at about
2^-16 of sum_d |q_d k_d|, where the bf16 instruction's is about 2^-22.  The
LSE bar (1e-3) is therefore claimed for score ranges where
scale * max_j sum_d |q_id k_jd| <= 32 (at most about 5e-4 of score error);
the N(0, 1) draws of the ordinary cases stay near 12, the wide-range case
checks on the CPU that its inputs stay inside it, and every case applies the
plain bars.  The score error also moves O: by at most
eps_i sum_j P_ij |V_jd - O_id| <= eps_i (sum_j P_ij |V_jd| + |O_id|), with
eps_i the row's largest score error; the wide-range case adds that term to
the O bound, with eps_i = 2^-15 scale max_j sum_d |q_id k_jd| (twice the
measured rate of the instruction)."""

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora

from gpu_helpers import TOL_LSE, max_abs, o_excess, say, scale_for, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa as _fa
    return _fa


def bytes_to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


FP8_CASES = [
    # (B, N, Hq, Hkv, d): one tile, ragged tails, GQA/MQA, a single token, several tiles
    (1, 128, 2, 2, 64),
    (1, 200, 2, 2, 64),
    (2, 333, 4, 4, 128),
    (1, 1, 2, 1, 128),
    (1, 17, 3, 1, 64),
    (2, 300, 8, 2, 128),
    (1, 1024, 4, 2, 128),
    (1, 777, 2, 2, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", FP8_CASES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_forward_parity(fa, shape, causal):
    import torch
    B, N, Hq, Hkv, d = shape
    say(f"fp8 fwd B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    x = inputs.fp8_dense_inputs(B, N, Hq, Hkv, d, seed=21)
    sc = scale_for(d)
    q8 = bytes_to_dev(x["q8"]).view(torch.float8_e4m3fn)   # both byte dtypes are accepted
    o, lse = fa.fwd_fp8(q8, bytes_to_dev(x["k8"]), to_dev(x["v"]), x["q_descale"],
                        x["k_descale"], causal=causal, softmax_scale=sc)
    ro, rlse = ora.attention_forward(x["q"], x["k"], x["v"], sc, causal)
    pv, _ = ora.attention_forward(x["q"], x["k"], np.abs(x["v"]), sc, causal)
    errs = dict(o=max_abs(to_host(o), ro), o_excess=o_excess(to_host(o), ro, pv, N),
                lse=max_abs(to_host(lse), rlse))
    say(f"errors {errs}")
    assert errs["o_excess"] <= 1.0
    assert errs["lse"] <= TOL_LSE


SCORE_RANGE = 32.0   # scale * max_j sum_d |q_id k_jd| up to which the LSE bar is claimed


def score_magnitude(q, k, G, scale, causal):
    """scale * max over visible keys of sum_d |q_id k_jd| per (head, row);
    q [N, Hq, d], k [N, Hkv, d]."""
    kk = np.repeat(k, G, axis=1)
    mag = np.einsum("ihd,jhd->hij", np.abs(q), np.abs(kk)) * scale
    if causal:
        n = q.shape[0]
        mag = np.where(np.tril(np.ones((n, n), dtype=bool)), mag, 0.0)
    return mag.max(axis=2)


def test_fp8_forward_wide_score_range(fa):
    """Descale factors 1.5 times the usual ones: scores up to about 11 in
    natural-log units (16 in log2 units), the widest range inside SCORE_RANGE."""
    say("fp8 fwd wide scores B=1 N=500 Hq=4 Hkv=2 d=128")
    x = inputs.fp8_dense_inputs(1, 500, 4, 2, 128, seed=22)
    f = 1.5
    qd, kd = x["q_descale"] * f, x["k_descale"] * f
    mag = score_magnitude(x["q"][0] * f, x["k"][0] * f, 2, scale_for(128), True)
    say(f"scale * max sum |q||k| = {float(mag.max()):.1f}")
    assert mag.max() <= SCORE_RANGE
    o, lse = fa.fwd_fp8(bytes_to_dev(x["q8"]), bytes_to_dev(x["k8"]), to_dev(x["v"]), qd, kd,
                        causal=True, softmax_scale=scale_for(128))
    ro, rlse = ora.attention_forward(x["q"] * f, x["k"] * f, x["v"], scale_for(128), True)
    pv, _ = ora.attention_forward(x["q"] * f, x["k"] * f, np.abs(x["v"]), scale_for(128), True)
    say(f"lse range {float(np.min(rlse)):.1f}..{float(np.max(rlse)):.1f}")
    # the instruction's score error moves O by at most eps_i (pv + |O*|)
    eps = 2.0 ** -15 * mag.T[None, :, :, None]                   # [1, N, Hq, 1]
    errs = dict(o_excess=o_excess(to_host(o), ro, pv, 500, extra=eps * (pv + np.abs(ro))),
                lse=max_abs(to_host(lse), rlse))
    say(f"errors {errs}")
    assert errs["o_excess"] <= 1.0 and errs["lse"] <= TOL_LSE


def test_fp8_forward_full_size(fa):
    """The benchmark's fp8 launch: B=2 H=16 N=8192 d=128 causal.  One whole
    head against the oracle, and sampled query rows (the first and last 32
    plus 96 random ones) of four more heads."""
    import torch
    B, N, H, d = 2, 8192, 16, 128
    say(f"fp8 fwd full size B={B} N={N} H={H} d={d} causal")
    x = inputs.fp8_dense_inputs(B, N, H, H, d, seed=23)
    sc = scale_for(d)
    o, lse = fa.fwd_fp8(bytes_to_dev(x["q8"]), bytes_to_dev(x["k8"]), to_dev(x["v"]),
                        x["q_descale"], x["k_descale"], causal=True, softmax_scale=sc)
    torch.cuda.synchronize()
    b, h = 1, 7
    sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
    ro, rlse = ora.attention_forward(x["q"][sl], x["k"][sl], x["v"][sl], sc, True)
    pv, _ = ora.attention_forward(x["q"][sl], x["k"][sl], np.abs(x["v"][sl]), sc, True)
    errs = dict(o_excess=o_excess(to_host(o[b:b + 1, :, h:h + 1]), ro, pv, N),
                lse=max_abs(to_host(lse[b:b + 1, h:h + 1]), rlse))
    say(f"whole head b={b} h={h} errors {errs}")
    assert errs["o_excess"] <= 1.0 and errs["lse"] <= TOL_LSE
    rng = np.random.Generator(np.random.PCG64(24))
    rows = np.unique(np.r_[np.arange(32), np.arange(N - 32, N), rng.integers(0, N, 96)])
    for (b, h) in ((0, 0), (0, 15), (1, 3), (1, 12)):
        qh, kh, vh = x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h]
        r_o, r_lse, _, _ = ora.head_query_rows(qh, kh, vh, np.zeros_like(vh), sc, True, rows)
        pv = ora.head_query_rows(qh, kh, np.abs(vh), np.zeros_like(vh), sc, True, rows)[0]
        e = dict(o_excess=o_excess(to_host(o[b, rows, h]), r_o, pv, N),
                 lse=max_abs(to_host(lse[b, h, rows]), r_lse))
        say(f"rows b={b} h={h} errors {e}")
        assert e["o_excess"] <= 1.0 and e["lse"] <= TOL_LSE


def lse_error(lse, ref) -> float:
    """Max |LSE - LSE*| over rows that see a key; rows that see none must be
    -inf on both sides (returns inf otherwise)."""
    empty = np.isneginf(ref)
    if not np.array_equal(np.isneginf(lse), empty):
        return float("inf")
    return float(np.max(np.abs(lse[~empty] - ref[~empty]))) if np.any(~empty) else 0.0


FP8_QK_CASES = [
    # (query lengths, key lengths, Hq, Hkv, d): decode rows and short chunks,
    # more queries than keys, empty sequences, split one-query tiles (more
    # than 32 key tiles of 64), chunked prefill
    ([1, 1, 3, 1, 17], [700, 33, 1029, 1, 260], 8, 2, 128),
    ([300, 64, 5, 40], [100, 64, 1, 700], 2, 2, 64),
    ([0, 7, 129, 1], [50, 0, 513, 257], 4, 1, 128),
    ([1, 17, 33, 289], [5000, 2049, 5000, 2100], 4, 2, 128),
    ([1, 3], [9000, 4100], 2, 1, 64),
    ([256, 257, 31], [1000, 600, 31], 4, 4, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", FP8_QK_CASES, ids=lambda c: f"n{len(c[0])}h{c[2]}{c[3]}d{c[4]}")
def test_fp8_varlen_qk_forward_parity(fa, case, causal):
    import torch
    lq, lk, Hq, Hkv, d = case
    say(f"fp8 varlen_qk lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    x = inputs.fp8_varlen_qk_inputs(lq, lk, Hq, Hkv, d, seed=len(lq) + d)
    cq = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    ck = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    sc = scale_for(d)
    o, lse = fa.varlen_qk_fwd_fp8(bytes_to_dev(x["q8"]), bytes_to_dev(x["k8"]), to_dev(x["v"]),
                                  cq, ck, x["q_descale"], x["k_descale"], causal=causal,
                                  softmax_scale=sc)
    o, lse = to_host(o), to_host(lse)
    ro, rlse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                     x["cu_seqlens_k"], sc, causal)
    pv, _ = ora.varlen_qk_forward(x["q"], x["k"], np.abs(x["v"]), x["cu_seqlens_q"],
                                  x["cu_seqlens_k"], sc, causal)
    errs = dict(o_excess=o_excess(o, ro, pv, max(lk)), lse=lse_error(lse, rlse))
    say(f"errors {errs}")
    assert np.all(np.isfinite(o))
    assert errs["o_excess"] <= 1.0 and errs["lse"] <= TOL_LSE
    empty = np.isneginf(rlse).T  # [Tq, Hq]: rows that see no key are exactly zero
    assert np.all(o[empty] == 0.0)
