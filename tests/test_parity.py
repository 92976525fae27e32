"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded bf16 inputs, element by element, at sizes that span several
tiles and ragged tails, plus GQA/MQA, packed variable-length batches and the
deterministic mode."""

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora

from gpu_helpers import (TOL_GRAD, TOL_LSE, max_abs, o_excess, rel_fro, say, scale_for, to_dev,
                         to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa as _fa
    return _fa


def run_dense(fa, B, N, Hq, Hkv, d, causal, seed=0, deterministic=False):
    say(f"dense B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal} det={deterministic} seed={seed}")
    x = inputs.dense_inputs(B, N, Hq, Hkv, d, seed=seed)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    sc = scale_for(d)
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=causal, softmax_scale=sc)
    dq, dk, dv = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal, softmax_scale=sc,
                        deterministic=deterministic)
    return x, t, (o, lse, dq, dk, dv)


def check_against_oracle(x, outs, causal, d):
    o, lse, dq, dk, dv = (to_host(a) for a in outs)
    sc = scale_for(d)
    ro, rlse = ora.attention_forward(x["q"], x["k"], x["v"], sc, causal)
    pv, _ = ora.attention_forward(x["q"], x["k"], np.abs(x["v"]), sc, causal)
    rdq, rdk, rdv = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], sc, causal)
    errs = dict(o=max_abs(o, ro), o_excess=o_excess(o, ro, pv, x["k"].shape[1]),
                lse=max_abs(lse, rlse),
                dq=rel_fro(dq, rdq), dk=rel_fro(dk, rdk), dv=rel_fro(dv, rdv))
    say(f"errors {errs}")
    assert errs["o_excess"] <= 1.0
    assert errs["lse"] <= TOL_LSE
    assert errs["dq"] <= TOL_GRAD
    assert errs["dk"] <= TOL_GRAD
    assert errs["dv"] <= TOL_GRAD


DENSE_CASES = [
    # (B, N, Hq, Hkv, d): the tiny configuration, ragged tails, GQA, MQA, single token
    (1, 128, 2, 2, 64),
    (1, 200, 2, 2, 64),
    (2, 333, 4, 4, 128),
    (1, 1, 2, 1, 128),
    (1, 17, 3, 1, 64),
    (2, 300, 8, 2, 128),
    (1, 260, 4, 1, 64),
    (1, 1024, 4, 2, 128),
    (1, 777, 2, 2, 128),
    # query tile 7 (rows 224..) holds the last rows: the fast mode's stored
    # tile 8m + 7 ends ragged
    (1, 250, 2, 2, 128),
    (2, 250, 3, 1, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", DENSE_CASES, ids=lambda s: "x".join(map(str, s)))
def test_dense_parity(fa, shape, causal):
    B, N, Hq, Hkv, d = shape
    x, _, outs = run_dense(fa, B, N, Hq, Hkv, d, causal)
    check_against_oracle(x, outs, causal, d)


HEAD256_CASES = [
    # d = 256: 256-row forward tiles, 128-key backward workgroups; ragged
    # tails on both, GQA/MQA, a single token
    (1, 300, 2, 1, 256),
    (2, 129, 4, 4, 256),
    (1, 1, 2, 2, 256),
    (1, 513, 4, 2, 256),
    (1, 257, 2, 2, 256),
]


@pytest.mark.parametrize("det", [0, 1], ids=["atomic", "ordered"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", HEAD256_CASES, ids=lambda s: "x".join(map(str, s)))
def test_head_dim_256_parity(fa, shape, causal, det):
    B, N, Hq, Hkv, d = shape
    x, _, outs = run_dense(fa, B, N, Hq, Hkv, d, causal, seed=11, deterministic=det)
    check_against_oracle(x, outs, causal, d)


def test_head_dim_256_ordered_is_bit_identical(fa):
    import torch
    x, t, outs = run_dense(fa, 1, 400, 4, 2, 256, True, seed=12, deterministic=1)
    ref = [a.clone() for a in outs[2:]]
    for rep in range(10):
        g = fa.bwd(t["q"], t["k"], t["v"], outs[0], outs[1], t["do"], causal=True,
                   softmax_scale=scale_for(256), deterministic=1)
        for a, b in zip(g, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), rep


@pytest.mark.parametrize("mode", [1, 2, 3], ids=["ordered", "partial", "fused"])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_parity_deterministic(fa, causal, mode):
    x, _, outs = run_dense(fa, 2, 451, 6, 2, 128, causal, seed=3, deterministic=mode)
    check_against_oracle(x, outs, causal, 128)


PARTIAL_CASES = [(1, 128, 2, 2, 64), (1, 1, 2, 1, 128), (1, 17, 3, 1, 64), (2, 300, 8, 2, 128),
                 (1, 1024, 4, 2, 128), (1, 777, 2, 2, 64)]


@pytest.mark.parametrize("mode", [2, 3], ids=["partial", "fused"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", PARTIAL_CASES, ids=lambda s: "x".join(map(str, s)))
def test_dense_parity_partial_sums(fa, shape, causal, mode):
    """dQ summed from per-(query tile, key tile) partial tiles, by a second
    kernel (mode 2) or by the last contributor inside the kernel (mode 3)."""
    B, N, Hq, Hkv, d = shape
    x, _, outs = run_dense(fa, B, N, Hq, Hkv, d, causal, seed=7, deterministic=mode)
    check_against_oracle(x, outs, causal, d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 513, 4, 2, 128), (1, 777, 2, 2, 64), (1, 1, 2, 1, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_partial_tile_modes_agree_bit_for_bit(fa, shape, causal):
    """Modes 2 and 3 add the same dQ partial tiles in the same order, so dQ
    agrees bit for bit.  (dK and dV agree too without a causal mask; with it,
    mode 3 walks the query tiles from the top, which changes the order of
    their register sums, so they only agree within rounding.)"""
    import torch
    B, N, Hq, Hkv, d = shape
    x, t, outs = run_dense(fa, B, N, Hq, Hkv, d, causal, seed=9, deterministic=2)
    g3 = fa.bwd(t["q"], t["k"], t["v"], outs[0], outs[1], t["do"], causal=causal,
                softmax_scale=scale_for(d), deterministic=3)
    assert torch.equal(outs[2].view(torch.int16), g3[0].view(torch.int16))
    for a, b in zip(outs[3:], g3[1:]):
        if causal:
            assert rel_fro(to_host(b), to_host(a)) <= 1e-2
        else:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("mode", [1, 2, 3], ids=["ordered", "partial", "fused"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 513, 4, 2, 128), (1, 640, 2, 1, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_deterministic_is_bit_identical(fa, shape, causal, mode):
    import torch
    B, N, Hq, Hkv, d = shape
    x, t, outs = run_dense(fa, B, N, Hq, Hkv, d, causal, seed=5, deterministic=mode)
    o, lse = outs[0], outs[1]
    ref = [a.clone() for a in outs[2:]]
    for rep in range(10):
        g = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal,
                   softmax_scale=scale_for(d), deterministic=mode)
        for a, b in zip(g, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), rep
    o2, lse2 = fa.fwd(t["q"], t["k"], t["v"], causal=causal, softmax_scale=scale_for(d))
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16))
    assert torch.equal(lse2, lse)


def test_forward_independent_of_tile_order(fa, monkeypatch):
    import torch
    x = inputs.dense_inputs(2, 700, 8, 2, 128, seed=2)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v")}
    o1, l1 = fa.fwd(t["q"], t["k"], t["v"], causal=True)
    monkeypatch.setenv("FA_SCHED", "natural")
    o2, l2 = fa.fwd(t["q"], t["k"], t["v"], causal=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_varlen_independent_of_tile_order(fa, monkeypatch):
    """The packed batch with the scheduler's cost sort switched off: the same
    forward and deterministic backward, bit for bit."""
    import torch
    lengths = [300, 1, 2500, 77, 1024]
    x = inputs.varlen_inputs(lengths, 4, 2, 128, seed=5)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    cu = torch.from_numpy(x["cu_seqlens"]).to("cuda")

    def run():
        o, lse = fa.varlen_fwd(t["q"], t["k"], t["v"], cu, causal=True)
        g = fa.varlen_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cu, causal=True,
                          deterministic=True)
        torch.cuda.synchronize()
        return (o, lse) + tuple(g)

    a = run()
    monkeypatch.setenv("FA_SCHED", "natural")
    b = run()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int32) if u.dtype == torch.float32 else u.view(torch.int16),
                           v.view(torch.int32) if v.dtype == torch.float32 else v.view(torch.int16))


def run_varlen(fa, lengths, Hq, Hkv, d, causal, deterministic=False, seed=0):
    import torch
    say(f"varlen lengths={lengths} Hq={Hq} Hkv={Hkv} d={d} causal={causal} det={deterministic}")
    x = inputs.varlen_inputs(lengths, Hq, Hkv, d, seed=seed)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    cu = torch.from_numpy(x["cu_seqlens"]).to("cuda")
    sc = scale_for(d)
    o, lse = fa.varlen_fwd(t["q"], t["k"], t["v"], cu, causal=causal, softmax_scale=sc)
    dq, dk, dv = fa.varlen_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cu, causal=causal,
                               softmax_scale=sc, deterministic=deterministic)
    return x, t, cu, (o, lse, dq, dk, dv)


VARLEN_CASES = [
    ([1, 5, 130, 257, 64, 600, 33], 4, 2, 128),
    ([300, 1, 1000, 129], 2, 2, 64),
    ([513], 3, 1, 128),
]


@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"n{len(c[0])}h{c[1]}{c[2]}d{c[3]}")
def test_varlen_parity(fa, case, causal, det):
    lengths, Hq, Hkv, d = case
    x, _, _, outs = run_varlen(fa, lengths, Hq, Hkv, d, causal, det)
    o, lse, dq, dk, dv = (to_host(a) for a in outs)
    sc = scale_for(d)
    cu = x["cu_seqlens"]
    ro, rlse = ora.varlen_forward(x["q"], x["k"], x["v"], cu, sc, causal)
    pv, _ = ora.varlen_forward(x["q"], x["k"], np.abs(x["v"]), cu, sc, causal)
    rdq, rdk, rdv = ora.varlen_backward(x["q"], x["k"], x["v"], x["do"], cu, sc, causal)
    errs = dict(o=max_abs(o, ro), o_excess=o_excess(o, ro, pv, max(lengths)),
                lse=max_abs(lse, rlse),
                dq=rel_fro(dq, rdq), dk=rel_fro(dk, rdk), dv=rel_fro(dv, rdv))
    say(f"errors {errs}")
    assert errs["o_excess"] <= 1.0 and errs["lse"] <= TOL_LSE
    assert errs["dq"] <= TOL_GRAD and errs["dk"] <= TOL_GRAD and errs["dv"] <= TOL_GRAD


def test_varlen_deterministic_bit_identical(fa):
    import torch
    lengths = [700, 3, 128, 1029, 64]
    x, t, cu, outs = run_varlen(fa, lengths, 4, 1, 128, True, deterministic=True, seed=4)
    o, lse = outs[0], outs[1]
    ref = [a.clone() for a in outs[2:]]
    for rep in range(10):
        g = fa.varlen_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cu, causal=True,
                          softmax_scale=scale_for(128), deterministic=True)
        for a, b in zip(g, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), rep


def test_varlen_bad_cu_seqlens_is_reported(fa):
    import torch
    say("varlen bad cu_seqlens")
    x = inputs.varlen_inputs([10, 20, 30], 2, 2, 64, seed=1)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v")}
    bad = torch.tensor([0, 20, 10, 60], dtype=torch.int32, device="cuda")  # decreasing
    ws = fa.varlen_fwd_workspace(3, 60, 2, 2, 64, True, "cuda")
    fa.varlen_fwd(t["q"], t["k"], t["v"], bad, causal=True, workspace=ws)
    assert fa.workspace_error(ws) & 1
    good = torch.from_numpy(x["cu_seqlens"]).to("cuda")
    fa.varlen_fwd(t["q"], t["k"], t["v"], good, causal=True, workspace=ws)
    assert fa.workspace_error(ws) == 0


def test_ordered_wait_timeout_is_reported(fa, monkeypatch):
    """A semaphore wait of the ordered dQ mode that outlasts its bound sets the
    device error bit and proceeds, so the kernel always exits and the call
    returns normally; the adds stay atomic, so dQ is still the right sum (only
    its bit-exact order is lost).  The bound is forced down to one tick of
    the 100 MHz clock from the host; non-causal rows make every key tile of a
    query tile wait for all the higher ones, so waits far beyond 64 polls
    occur."""
    import torch
    B, N, Hq, d = 1, 4096, 4, 128
    say(f"ordered wait timeout B={B} N={N} Hq={Hq} d={d} non-causal")
    x = inputs.dense_inputs(B, N, Hq, Hq, d, seed=41)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    sc = scale_for(d)
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=False, softmax_scale=sc)
    ref = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=False, softmax_scale=sc,
                 deterministic=0)
    monkeypatch.setenv("FA_DET_SPIN_TICKS", "1")
    ws = fa.bwd_workspace(t["q"], t["k"], False, 1)
    g = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=False, softmax_scale=sc,
               deterministic=1, workspace=ws)
    torch.cuda.synchronize()
    bits = fa.workspace_error(ws)
    monkeypatch.delenv("FA_DET_SPIN_TICKS")
    errs = {n: rel_fro(to_host(a), to_host(b)) for n, a, b in zip(("dq", "dk", "dv"), g, ref)}
    say(f"error bits {bits}, against the atomic mode {errs}")
    assert bits & 2
    # dK, dV never depend on the dQ order; dQ differs from the atomic mode's
    # only by the order of its fp32 adds (a few bf16 roundings)
    assert errs["dk"] <= 1e-6 and errs["dv"] <= 1e-6 and errs["dq"] <= 1e-2
    # with the default bound the same call reports nothing
    g = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=False, softmax_scale=sc,
               deterministic=1, workspace=ws)
    assert fa.workspace_error(ws) == 0
