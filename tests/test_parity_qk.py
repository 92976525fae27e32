"""GPU parity of the packed path with separate query and key lengths (decode
and chunked-prefill shaped batches, bottom-right causal alignment) against
the fp64 oracle, through the C ABI: element by element on small batches with
ragged tails, empty rows and empty sequences; sampled rows and keys of every
sequence on the full-size decode-shaped batch."""

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora

from gpu_helpers import TOL_GRAD, TOL_LSE, o_excess, rel_fro, say, scale_for, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa as _fa
    return _fa


def run_qk(fa, lq, lk, Hq, Hkv, d, causal, deterministic=0, seed=0):
    import torch
    say(f"varlen_qk lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} det={deterministic}")
    x = inputs.varlen_qk_inputs(lq, lk, Hq, Hkv, d, seed=seed)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    cq = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    ck = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    sc = scale_for(d)
    o, lse = fa.varlen_qk_fwd(t["q"], t["k"], t["v"], cq, ck, causal=causal, softmax_scale=sc)
    dq, dk, dv = fa.varlen_qk_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=causal,
                                  softmax_scale=sc, deterministic=deterministic)
    return x, t, (cq, ck), (o, lse, dq, dk, dv)


def lse_error(lse, ref) -> float:
    """Max |LSE - LSE*| over rows that see a key; rows that see none must be
    -inf on both sides (returns inf otherwise)."""
    empty = np.isneginf(ref)
    if not np.array_equal(np.isneginf(lse), empty):
        return float("inf")
    return float(np.max(np.abs(lse[~empty] - ref[~empty]))) if np.any(~empty) else 0.0


QK_CASES = [
    # (query lengths, key lengths, Hq, Hkv, d)
    ([1, 1, 3, 1, 17], [700, 33, 1029, 1, 260], 8, 2, 128),   # decode rows and short chunks
    ([300, 64, 5, 40], [100, 64, 1, 700], 2, 2, 64),           # more queries than keys
    ([0, 7, 129, 1], [50, 0, 513, 257], 4, 1, 128),            # empty sequences
    ([256, 257, 31], [1000, 600, 31], 4, 4, 64),               # chunked prefill
    ([1, 130, 40, 0], [300, 129, 20, 17], 2, 1, 256),          # d = 256
]


@pytest.mark.parametrize("det", [0, 1])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", QK_CASES, ids=lambda c: f"n{len(c[0])}h{c[2]}{c[3]}d{c[4]}")
def test_varlen_qk_parity(fa, case, causal, det):
    lq, lk, Hq, Hkv, d = case
    x, _, _, outs = run_qk(fa, lq, lk, Hq, Hkv, d, causal, det, seed=len(lq) + d)
    o, lse, dq, dk, dv = (to_host(a) for a in outs)
    sc = scale_for(d)
    ro, rlse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                     x["cu_seqlens_k"], sc, causal)
    rdq, rdk, rdv = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                                           x["cu_seqlens_k"], sc, causal)
    pv, _ = ora.varlen_qk_forward(x["q"], x["k"], np.abs(x["v"]), x["cu_seqlens_q"],
                                  x["cu_seqlens_k"], sc, causal)
    errs = dict(o_excess=o_excess(o, ro, pv, max(lk)), lse=lse_error(lse, rlse),
                dq=rel_fro(dq, rdq),
                dk=rel_fro(dk, rdk), dv=rel_fro(dv, rdv))
    say(f"errors {errs}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(dq))
    assert np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    assert errs["o_excess"] <= 1.0 and errs["lse"] <= TOL_LSE
    assert errs["dq"] <= TOL_GRAD and errs["dk"] <= TOL_GRAD and errs["dv"] <= TOL_GRAD
    # rows that see no key: exactly zero output and query gradient
    empty = np.isneginf(rlse).T  # [Tq, Hq]
    assert np.all(o[empty] == 0.0) and np.all(dq[empty] == 0.0)


SPLIT_CASES = [
    # last query tile with <= 32 rows against more than 32 key tiles: split
    # into chunks of 32 key tiles and merged by the combine kernel
    ([1, 17, 32, 33, 257, 288, 289], [5000, 5000, 2049, 5000, 3000, 2100, 2100], 4, 2, 128),
    ([1, 3], [70000, 4100], 2, 1, 64),
    ([1, 257, 288], [4500, 3000, 2100], 2, 2, 256),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: f"n{len(c[0])}d{c[4]}")
def test_split_query_tiles(fa, case, causal):
    lq, lk, Hq, Hkv, d = case
    x, _, _, outs = run_qk(fa, lq, lk, Hq, Hkv, d, causal, 0, seed=7)
    o, lse = to_host(outs[0]), to_host(outs[1])
    sc = scale_for(d)
    ro, rlse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                     x["cu_seqlens_k"], sc, causal)
    pv, _ = ora.varlen_qk_forward(x["q"], x["k"], np.abs(x["v"]), x["cu_seqlens_q"],
                                  x["cu_seqlens_k"], sc, causal)
    errs = dict(o_excess=o_excess(o, ro, pv, max(lk)), lse=lse_error(lse, rlse))
    rdq, rdk, rdv = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                                           x["cu_seqlens_k"], sc, causal)
    dq, dk, dv = (to_host(a) for a in outs[2:])
    errs.update(dq=rel_fro(dq, rdq), dk=rel_fro(dk, rdk), dv=rel_fro(dv, rdv))
    say(f"errors {errs}")
    assert errs["o_excess"] <= 1.0 and errs["lse"] <= TOL_LSE
    assert errs["dq"] <= TOL_GRAD and errs["dk"] <= TOL_GRAD and errs["dv"] <= TOL_GRAD


def test_split_tiles_in_equal_length_batches(fa):
    """The single-offset packed forward splits too (a 2305-token sequence
    ends with a one-row tile over 37 key tiles); repeated calls agree bit
    for bit."""
    import torch
    lengths = [2305, 40, 4097]
    x = inputs.varlen_inputs(lengths, 2, 2, 128, seed=2)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v")}
    cu = torch.from_numpy(x["cu_seqlens"]).to("cuda")
    o, lse = fa.varlen_fwd(t["q"], t["k"], t["v"], cu, causal=True, softmax_scale=scale_for(128))
    o2, lse2 = fa.varlen_fwd(t["q"], t["k"], t["v"], cu, causal=True, softmax_scale=scale_for(128))
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    ro, rlse = ora.varlen_forward(x["q"], x["k"], x["v"], x["cu_seqlens"], scale_for(128), True)
    pv, _ = ora.varlen_forward(x["q"], x["k"], np.abs(x["v"]), x["cu_seqlens"], scale_for(128),
                               True)
    oe = o_excess(to_host(o), ro, pv, max(lengths))
    say(f"o_excess {oe:.3f} lse {lse_error(to_host(lse), rlse):.2e}")
    assert oe <= 1.0 and lse_error(to_host(lse), rlse) <= TOL_LSE


def test_equal_lengths_match_the_single_offset_call(fa):
    """With cu_seqlens_q == cu_seqlens_k the separate-length entry points run
    the same kernels on the same schedule: bit-identical forward and
    deterministic backward."""
    import torch
    lengths = [700, 3, 128, 1029, 64]
    x, t, (cq, ck), outs = run_qk(fa, lengths, lengths, 4, 2, 128, True, deterministic=1, seed=4)
    o2, lse2 = fa.varlen_fwd(t["q"], t["k"], t["v"], cq, causal=True, softmax_scale=scale_for(128))
    g2 = fa.varlen_bwd(t["q"], t["k"], t["v"], o2, lse2, t["do"], cq, causal=True,
                       softmax_scale=scale_for(128), deterministic=True)
    assert torch.equal(outs[0].view(torch.int16), o2.view(torch.int16))
    assert torch.equal(outs[1], lse2)
    for a, b in zip(outs[2:], g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_varlen_qk_deterministic_bit_identical(fa):
    import torch
    lq, lk = [1, 64, 300, 17, 2], [900, 64, 1200, 3, 700]
    x, t, (cq, ck), outs = run_qk(fa, lq, lk, 4, 1, 128, True, deterministic=1, seed=8)
    o, lse = outs[0], outs[1]
    ref = [a.clone() for a in outs[2:]]
    for rep in range(10):
        g = fa.varlen_qk_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=True,
                             softmax_scale=scale_for(128), deterministic=1)
        for a, b in zip(g, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), rep


def test_varlen_qk_bad_key_offsets_are_reported(fa):
    import torch
    say("varlen_qk bad cu_seqlens_k")
    x = inputs.varlen_qk_inputs([3, 4], [10, 20], 2, 2, 64, seed=1)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v")}
    cq = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    bad = torch.tensor([0, 10, 25], dtype=torch.int32, device="cuda")  # last != total_k
    ws = fa.varlen_qk_fwd_workspace(2, 7, 30, 2, 2, 64, True, "cuda")
    fa.varlen_qk_fwd(t["q"], t["k"], t["v"], cq, bad, causal=True, workspace=ws)
    assert fa.workspace_error(ws) & 1
    good = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    fa.varlen_qk_fwd(t["q"], t["k"], t["v"], cq, good, causal=True, workspace=ws)
    assert fa.workspace_error(ws) == 0


# ---------------------------------------------------------------------------
# full size: the decode-shaped batch (65536 keys in log-uniform sequences of
# 128..16384 tokens, half the sequences one query, the rest a chunk of up to
# 1024 queries), Hq = 32, Hkv = 4, d = 128, causal, in the benchmark's launch
# configuration; sampled rows and the last keys of every sequence.

QK_HQ, QK_HKV, QK_D = 32, 4, 128


@pytest.fixture(scope="module")
def qk_problem(fa):
    import torch
    lq, lk = inputs.qk_lengths()
    x = inputs.varlen_qk_inputs(lq, lk, QK_HQ, QK_HKV, QK_D, seed=0)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    cq = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    ck = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    return x, t, cq, ck, lq, lk


@pytest.mark.parametrize("det", [0, 1])
def test_decode_batch_full_size(fa, qk_problem, det):
    x, t, cq, ck, lq, lk = qk_problem
    say(f"decode batch nseq={len(lq)} Tq={sum(lq)} Tk={sum(lk)} det={det}")
    sc = scale_for(QK_D)
    o, lse = fa.varlen_qk_fwd(t["q"], t["k"], t["v"], cq, ck, causal=True, softmax_scale=sc)
    dq, dk, dv = fa.varlen_qk_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=True,
                                  softmax_scale=sc, deterministic=det)
    o, lse, dq, dk, dv = (to_host(a) for a in (o, lse, dq, dk, dv))
    G = QK_HQ // QK_HKV
    rng = np.random.Generator(np.random.PCG64(17))
    cu_q, cu_k = x["cu_seqlens_q"], x["cu_seqlens_k"]
    worst = dict(o_excess=0.0, lse=0.0, dq=0.0, dk=0.0, dv=0.0)
    for s in range(len(lq)):
        qa, qe, ka, ke = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        off = (ke - ka) - (qe - qa)
        rows = np.unique(np.concatenate([[0, qe - qa - 1], rng.integers(0, qe - qa, 2)]))
        keys = np.unique(np.concatenate([[0, ke - ka - 1], rng.integers(0, ke - ka, 2)]))
        g = int(rng.integers(0, QK_HKV))
        kh, vh = x["k"][ka:ke, g], x["v"][ka:ke, g]
        dk_ref = np.zeros((keys.size, QK_D))
        dv_ref = np.zeros((keys.size, QK_D))
        for h in range(g * G, (g + 1) * G):
            qh, doh = x["q"][qa:qe, h], x["do"][qa:qe, h]
            ro, rl, _, rdq = ora.head_query_rows(qh, kh, vh, doh, sc, True, rows, offset=off)
            pv = ora.head_query_rows(qh, kh, np.abs(vh), doh, sc, True, rows, offset=off)[0]
            worst["o_excess"] = max(worst["o_excess"], o_excess(o[qa + rows, h], ro, pv, ke - ka))
            worst["lse"] = max(worst["lse"], lse_error(lse[h, qa + rows], rl))
            worst["dq"] = max(worst["dq"], rel_fro(dq[qa + rows, h], rdq))
            a, b = ora.head_key_rows(qh, kh, vh, doh, sc, True, keys, offset=off)
            dk_ref += a
            dv_ref += b
        worst["dk"] = max(worst["dk"], rel_fro(dk[ka + keys, g], dk_ref))
        worst["dv"] = max(worst["dv"], rel_fro(dv[ka + keys, g], dv_ref))
    say(f"worst {worst}")
    assert worst["o_excess"] <= 1.0 and worst["lse"] <= TOL_LSE
    assert worst["dq"] <= TOL_GRAD and worst["dk"] <= TOL_GRAD and worst["dv"] <= TOL_GRAD
    # sum over keys of dV equals sum over queries (and the group's heads) of dO,
    # per sequence and key/value head (every query here sees a key: Lq <= Lk);
    # it holds at any size
    for s in range(len(lq)):
        qa, qe, ka, ke = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        lhs = dv[ka:ke].sum(axis=0)
        rhs = x["do"][qa:qe].astype(np.float64).sum(axis=0).reshape(QK_HKV, G, QK_D).sum(axis=1)
        err = float(np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs))
        assert err <= 1e-2, (s, err)
