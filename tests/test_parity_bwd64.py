"""GPU parity of the backward build with 64 keys per wave at d = 64 (4 waves
of two 32-key blocks each, one wave per SIMD; the variant `bwd64keys`,
built beside the library): the same products as the default 8-wave build in
the same order, so its dK and dV are bit-identical to the default's in every
mode and its dQ too in the ordered mode; the fast mode's dQ differs only in
the order of its fp32 atomic adds.  Each case is also held to the oracle at
the usual bars, and the partial-tile modes, which this build does not offer,
are refused."""

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora

from gpu_helpers import TOL_GRAD, rel_fro, say, scale_for, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa
    return fa, fa.load_variant("bwd64keys")


DENSE = [(1, 200, 2, 2), (2, 333, 4, 2), (1, 1, 2, 1), (1, 1000, 4, 4)]


def same(a, b) -> bool:
    import torch
    return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))


@pytest.mark.parametrize("det", [0, 1], ids=["atomic", "ordered"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", DENSE, ids=lambda s: "x".join(map(str, s)))
def test_dense_matches_default_build_and_oracle(libs, shape, causal, det):
    import torch
    fa, L = libs
    B, N, Hq, Hkv = shape
    say(f"bwd64keys dense B={B} N={N} Hq={Hq} Hkv={Hkv} causal={causal} det={det}")
    x = inputs.dense_inputs(B, N, Hq, Hkv, 64, seed=51)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    sc = scale_for(64)
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=causal, softmax_scale=sc)
    g0 = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal, softmax_scale=sc,
                deterministic=det)
    g1 = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal, softmax_scale=sc,
                deterministic=det, lib=L)
    torch.cuda.synchronize()
    assert same(g0[1], g1[1]) and same(g0[2], g1[2])
    if det == 1:
        assert same(g0[0], g1[0])
    rg = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], sc, causal)
    errs = {n: rel_fro(to_host(a), r) for n, a, r in zip(("dq", "dk", "dv"), g1, rg)}
    say(f"errors {errs}")
    assert max(errs.values()) <= TOL_GRAD


@pytest.mark.parametrize("det", [0, 1], ids=["atomic", "ordered"])
def test_packed_with_separate_lengths(libs, det):
    import torch
    fa, L = libs
    lq, lk = [1, 300, 0, 65, 7], [700, 300, 40, 129, 1]
    say(f"bwd64keys varlen_qk lq={lq} lk={lk} det={det}")
    x = inputs.varlen_qk_inputs(lq, lk, 4, 2, 64, seed=52)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    cq = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    ck = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    sc = scale_for(64)
    o, lse = fa.varlen_qk_fwd(t["q"], t["k"], t["v"], cq, ck, causal=True, softmax_scale=sc)
    g0 = fa.varlen_qk_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=True,
                          softmax_scale=sc, deterministic=det)
    g1 = fa.varlen_qk_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=True,
                          softmax_scale=sc, deterministic=det, lib=L)
    torch.cuda.synchronize()
    assert same(g0[1], g1[1]) and same(g0[2], g1[2])
    if det == 1:
        assert same(g0[0], g1[0])
    rg = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                                x["cu_seqlens_k"], sc, True)
    errs = {n: rel_fro(to_host(a), r) for n, a, r in zip(("dq", "dk", "dv"), g1, rg)}
    say(f"errors {errs}")
    assert max(errs.values()) <= TOL_GRAD


def test_partial_tile_modes_are_refused(libs):
    fa, L = libs
    x = inputs.dense_inputs(1, 128, 2, 2, 64, seed=53)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=True)
    for det in (2, 3):
        assert L.fa_bwd_workspace_size(1, 128, 2, 2, 64, 1, det) == 0
        with pytest.raises(fa.FAError, match="UNSUPPORTED"):
            fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=True, deterministic=det,
                   workspace=fa.bwd_workspace(t["q"], t["k"], True, det), lib=L)
