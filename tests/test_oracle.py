"""Pins for the CPU oracle: invariants, closed forms, finite differences and an
independent library implementation.  None of these re-types the oracle's own
formulas; each would catch a dropped term, a wrong sign or index, or a
transposed operand somewhere in the oracle.
"""

import json
import math
import os

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# The tiny configuration: B=1, H=2, N=128, d=64, fp32 N(0,1), scale 1/sqrt(d).
B0, H0, N0, D0 = 1, 2, 128, 64
SCALE0 = 1.0 / math.sqrt(D0)


@pytest.fixture(scope="module")
def tiny():
    return inputs.dense_inputs(B0, N0, H0, H0, D0, seed=0, round_bf16=False)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(tiny, causal):
    p = ora.attention_probs(tiny["q"], tiny["k"], SCALE0, causal)
    assert np.max(np.abs(p.sum(axis=-1) - 1.0)) <= 1e-12
    assert np.all(p >= 0)
    if causal:
        i, j = np.triu_indices(N0, k=1)
        assert np.all(p[..., i, j] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_output(tiny, causal):
    rng = np.random.Generator(np.random.PCG64(7))
    c = rng.standard_normal((B0, 1, H0, D0))
    v = np.broadcast_to(c, (B0, N0, H0, D0)).copy()
    o, _ = ora.attention_forward(tiny["q"], tiny["k"], v, SCALE0, causal)
    assert np.max(np.abs(o - c)) <= 1e-12


def test_causal_row_zero_sees_only_key_zero(tiny):
    q, k, v = (tiny[x].astype(np.float64) for x in ("q", "k", "v"))
    o, lse = ora.attention_forward(q, k, v, SCALE0, True)
    p = ora.attention_probs(q, k, SCALE0, True)
    assert np.all(p[:, :, 0, 0] == 1.0)
    assert np.max(np.abs(o[:, 0] - v[:, 0])) <= 1e-14
    expect = SCALE0 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0])
    assert np.max(np.abs(lse[:, :, 0] - expect)) <= 1e-12


def test_single_token_closed_form():
    x = inputs.dense_inputs(2, 1, 3, 3, 16, seed=3, round_bf16=False)
    q, k, v = (x[n].astype(np.float64) for n in ("q", "k", "v"))
    for causal in (False, True):
        o, lse = ora.attention_forward(q, k, v, 0.3, causal)
        assert np.max(np.abs(o - v)) <= 1e-15
        assert np.max(np.abs(lse - 0.3 * np.einsum("bnhd,bnhd->bhn", q, k))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_uniform_weights(tiny, causal):
    v = tiny["v"].astype(np.float64)
    q = np.zeros_like(tiny["q"], dtype=np.float64)
    o, lse = ora.attention_forward(q, tiny["k"], v, SCALE0, causal)
    n = np.arange(1, N0 + 1, dtype=np.float64)
    if causal:
        expect_o = np.cumsum(v, axis=1) / n[None, :, None, None]
        expect_lse = np.broadcast_to(np.log(n), lse.shape)
    else:
        expect_o = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
        expect_lse = np.full(lse.shape, math.log(N0))
    assert np.max(np.abs(o - expect_o)) <= 1e-12
    assert np.max(np.abs(lse - expect_lse)) <= 1e-12


def _golden():
    with open(os.path.join(GOLDEN, "two_token_closed_form.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("mode", ["non_causal", "causal"])
def test_two_token_closed_form(mode):
    g = _golden()
    a = {n: np.array(g["inputs"][n], dtype=np.float64)[None, :, None, :]
         for n in ("q", "k", "v", "do")}
    causal = mode == "causal"
    o, lse = ora.attention_forward(a["q"], a["k"], a["v"], g["inputs"]["scale"], causal)
    dq, dk, dv = ora.attention_backward(a["q"], a["k"], a["v"], a["do"],
                                        g["inputs"]["scale"], causal)
    e = g[mode]
    np.testing.assert_allclose(o[0, :, 0], e["o"], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], e["lse"], atol=1e-14)
    np.testing.assert_allclose(dq[0, :, 0], e["dq"], atol=1e-14)
    np.testing.assert_allclose(dk[0, :, 0], e["dk"], atol=1e-14)
    np.testing.assert_allclose(dv[0, :, 0], e["dv"], atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha_with_repeated_kv(causal):
    x = inputs.dense_inputs(2, 40, 6, 2, 8, seed=11, round_bf16=False)
    G = 3
    k_rep = np.repeat(x["k"], G, axis=2)
    v_rep = np.repeat(x["v"], G, axis=2)
    o_g, lse_g = ora.attention_forward(x["q"], x["k"], x["v"], 0.4, causal)
    o_m, lse_m = ora.attention_forward(x["q"], k_rep, v_rep, 0.4, causal)
    assert np.max(np.abs(o_g - o_m)) <= 1e-12
    assert np.max(np.abs(lse_g - lse_m)) <= 1e-12
    dq_g, dk_g, dv_g = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], 0.4, causal)
    dq_m, dk_m, dv_m = ora.attention_backward(x["q"], k_rep, v_rep, x["do"], 0.4, causal)
    assert np.max(np.abs(dq_g - dq_m)) <= 1e-12
    dk_sum = dk_m.reshape(2, 40, 2, G, 8).sum(axis=3)
    dv_sum = dv_m.reshape(2, 40, 2, G, 8).sum(axis=3)
    assert np.max(np.abs(dk_g - dk_sum)) <= 1e-12
    assert np.max(np.abs(dv_g - dv_sum)) <= 1e-12


def _objective(q, k, v, do, causal):
    o, _ = ora.attention_forward(q, k, v, SCALE0, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences(tiny, causal):
    """f = <O, dO>; its gradient w.r.t. Q, K, V is (dQ, dK, dV)."""
    x = {n: tiny[n].astype(np.float64) for n in ("q", "k", "v", "do")}
    dq, dk, dv = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], SCALE0, causal)
    grads = {"q": dq, "k": dk, "v": dv}
    rng = np.random.Generator(np.random.PCG64(5))
    h = 1e-5
    for name in ("q", "k", "v"):
        dirs = [rng.standard_normal(x[name].shape) for _ in range(8)]
        for _ in range(32):
            e = np.zeros(x[name].shape)
            e[tuple(rng.integers(0, s) for s in x[name].shape)] = 1.0
            dirs.append(e)
        for u in dirs:
            plus = dict(x)
            minus = dict(x)
            plus[name] = x[name] + h * u
            minus[name] = x[name] - h * u
            fd = (_objective(plus["q"], plus["k"], plus["v"], x["do"], causal)
                  - _objective(minus["q"], minus["k"], minus["v"], x["do"], causal)) / (2 * h)
            an = float(np.sum(grads[name] * u))
            scale_ref = max(1.0, abs(an), float(np.sqrt(np.sum(grads[name] ** 2))))
            assert abs(fd - an) <= 1e-6 * scale_ref, (name, fd, an)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sum_identities(tiny, causal):
    """Rows of dS sum to zero, so dK sums to zero over keys; rows of P sum to one,
    so dV summed over keys equals dO summed over queries (per head group)."""
    x = inputs.dense_inputs(2, 96, 4, 2, 32, seed=9, round_bf16=False)
    dq, dk, dv = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], 0.2, causal)
    assert np.max(np.abs(dk.sum(axis=1))) <= 1e-10
    do_sum = x["do"].astype(np.float64).sum(axis=1).reshape(2, 2, 2, 32).sum(axis=2)
    assert np.max(np.abs(dv.sum(axis=1) - do_sum)) <= 1e-10


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_fp64(tiny, causal):
    """Independent implementation: torch CPU float64 softmax + autograd."""
    torch = pytest.importorskip("torch")
    t = {n: torch.tensor(tiny[n], dtype=torch.float64) for n in ("q", "k", "v", "do")}
    q = t["q"].clone().requires_grad_(True)
    k = t["k"].clone().requires_grad_(True)
    v = t["v"].clone().requires_grad_(True)
    qh, kh, vh = (a.permute(0, 2, 1, 3) for a in (q, k, v))
    s = torch.matmul(qh, kh.transpose(-1, -2).contiguous()) * SCALE0
    if causal:
        mask = torch.triu(torch.ones(N0, N0, dtype=torch.bool), diagonal=1)
        s = s.masked_fill(mask, float("-inf"))
    lse_t = torch.logsumexp(s, dim=-1)
    o_t = torch.matmul(torch.softmax(s, dim=-1), vh).permute(0, 2, 1, 3)
    (o_t * t["do"]).sum().backward()
    o, lse = ora.attention_forward(tiny["q"], tiny["k"], tiny["v"], SCALE0, causal)
    dq, dk, dv = ora.attention_backward(tiny["q"], tiny["k"], tiny["v"], tiny["do"], SCALE0, causal)
    assert np.max(np.abs(o - o_t.detach().numpy())) <= 1e-12
    assert np.max(np.abs(lse - lse_t.detach().numpy())) <= 1e-12
    assert np.max(np.abs(dq - q.grad.numpy())) <= 1e-12
    assert np.max(np.abs(dk - k.grad.numpy())) <= 1e-12
    assert np.max(np.abs(dv - v.grad.numpy())) <= 1e-12


def test_joint_key_permutation_invariance(tiny):
    perm = np.random.Generator(np.random.PCG64(2)).permutation(N0)
    o1, lse1 = ora.attention_forward(tiny["q"], tiny["k"], tiny["v"], SCALE0, False)
    o2, lse2 = ora.attention_forward(tiny["q"], tiny["k"][:, perm], tiny["v"][:, perm], SCALE0, False)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(lse1 - lse2)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_scale_equivariance(tiny, causal):
    a = 2.5
    q = tiny["q"].astype(np.float64)
    o1, lse1 = ora.attention_forward(q, tiny["k"], tiny["v"], SCALE0, causal)
    o2, lse2 = ora.attention_forward(q / a, tiny["k"], tiny["v"], SCALE0 * a, causal)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(lse1 - lse2)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_row_chunking_is_exact(causal):
    x = inputs.dense_inputs(1, 100, 2, 1, 16, seed=4, round_bf16=False)
    full = ora.attention_forward(x["q"], x["k"], x["v"], 0.25, causal)
    chunked = ora.attention_forward(x["q"], x["k"], x["v"], 0.25, causal, row_chunk=7)
    for a, b in zip(full, chunked):
        assert np.max(np.abs(a - b)) <= 1e-13
    g_full = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], 0.25, causal)
    g_ch = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], 0.25, causal, row_chunk=7)
    for a, b in zip(g_full, g_ch):
        assert np.max(np.abs(a - b)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_uniform_lengths_match_dense_layout(causal):
    B, N, Hq, Hkv, d = 3, 24, 4, 2, 8
    x = inputs.dense_inputs(B, N, Hq, Hkv, d, seed=6, round_bf16=False)
    o, lse = ora.attention_forward(x["q"], x["k"], x["v"], 0.3, causal)
    dq, dk, dv = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], 0.3, causal)
    cu = inputs.cu_seqlens([N] * B)
    pk = {n: x[n].reshape(B * N, -1, d) for n in ("q", "k", "v", "do")}
    ov, lsev = ora.varlen_forward(pk["q"], pk["k"], pk["v"], cu, 0.3, causal)
    dqv, dkv, dvv = ora.varlen_backward(pk["q"], pk["k"], pk["v"], pk["do"], cu, 0.3, causal)
    assert np.max(np.abs(ov - o.reshape(B * N, Hq, d))) <= 1e-14
    assert np.max(np.abs(lsev - lse.transpose(1, 0, 2).reshape(Hq, B * N))) <= 1e-14
    assert np.max(np.abs(dqv - dq.reshape(B * N, Hq, d))) <= 1e-14
    assert np.max(np.abs(dkv - dk.reshape(B * N, Hkv, d))) <= 1e-14
    assert np.max(np.abs(dvv - dv.reshape(B * N, Hkv, d))) <= 1e-14


def test_varlen_sequences_are_independent():
    """Changing one sequence's keys leaves every other sequence untouched."""
    lengths = [5, 17, 1, 9]
    x = inputs.varlen_inputs(lengths, 2, 1, 8, seed=8)
    cu = x["cu_seqlens"]
    o1, _ = ora.varlen_forward(x["q"], x["k"], x["v"], cu, 0.5, True)
    k2 = x["k"].copy()
    k2[cu[1]:cu[2]] += np.random.Generator(np.random.PCG64(1)).standard_normal(k2[cu[1]:cu[2]].shape)
    o2, _ = ora.varlen_forward(x["q"], k2, x["v"], cu, 0.5, True)
    assert np.array_equal(o1[:cu[1]], o2[:cu[1]])
    assert np.array_equal(o1[cu[2]:], o2[cu[2]:])
    assert not np.allclose(o1[cu[1]:cu[2]], o2[cu[1]:cu[2]])
    # a length-1 sequence attends only to itself
    s = 2
    np.testing.assert_allclose(o1[cu[s]], np.repeat(x["v"][cu[s]], 2, axis=0), atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_moves_only_the_logsumexp(tiny, causal):
    """Adding one vector c to every key adds scale*q_i.c to every score of row i:
    P and O are unchanged and the logsumexp moves by exactly that amount."""
    c = np.random.Generator(np.random.PCG64(3)).standard_normal((1, 1, H0, D0))
    k2 = tiny["k"].astype(np.float64) + c
    o1, lse1 = ora.attention_forward(tiny["q"], tiny["k"], tiny["v"], SCALE0, causal)
    o2, lse2 = ora.attention_forward(tiny["q"], k2, tiny["v"], SCALE0, causal)
    shift = SCALE0 * np.einsum("bnhd,bhd->bhn", tiny["q"].astype(np.float64), c[:, 0])
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(lse2 - lse1 - shift)) <= 1e-12


def test_flop_convention():
    f, b = ora.attention_flops(2, 8192, 16, 128, True)
    assert f == 4 * 2 * 16 * 8192 ** 2 * 128 / 2
    assert b == 2.5 * f


def _torch_reference(q, k, v, do, scale, causal):
    """torch CPU float64 explicit softmax + autograd on one head pair."""
    import torch
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=(n != "do"))
         for n, a in (("q", q), ("k", k), ("v", v), ("do", do))}
    s = scale * t["q"] @ t["k"].T
    if causal:
        n = q.shape[0]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(s, dim=1)
    o = torch.softmax(s, dim=1) @ t["v"]
    (o * t["do"]).sum().backward()
    return (o.detach().numpy(), lse.detach().numpy(), t["q"].grad.numpy(),
            t["k"].grad.numpy(), t["v"].grad.numpy())


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_and_keys_match_autograd(causal):
    """The spot-check routines (chosen query rows; chosen keys, summed over a
    query-head group) against an independent torch float64 autograd."""
    pytest.importorskip("torch")
    x = inputs.dense_inputs(1, 150, 3, 1, 32, seed=11, round_bf16=False)
    q, k, v, do = (x[n][0].astype(np.float64) for n in ("q", "k", "v", "do"))
    scale = 0.17
    rows = np.array([0, 1, 63, 64, 100, 149, 5])
    keys = np.array([149, 0, 77, 3, 120])
    dk_sum = np.zeros((keys.size, 32))
    dv_sum = np.zeros((keys.size, 32))
    for h in range(3):
        ro, rlse, rdq, rdk, rdv = _torch_reference(q[:, h], k[:, 0], v[:, 0], do[:, h], scale,
                                                   causal)
        o, lse, dvec, dq = ora.head_query_rows(q[:, h], k[:, 0], v[:, 0], do[:, h], scale,
                                               causal, rows)
        assert np.max(np.abs(o - ro[rows])) <= 1e-12
        assert np.max(np.abs(lse - rlse[rows])) <= 1e-12
        assert np.max(np.abs(dvec - (ro[rows] * do[rows, h]).sum(axis=1))) <= 1e-12
        assert np.max(np.abs(dq - rdq[rows])) <= 1e-12
        dk, dv = ora.head_key_rows(q[:, h], k[:, 0], v[:, 0], do[:, h], scale, causal, keys,
                                   row_chunk=7)
        assert np.max(np.abs(dk - rdk[keys])) <= 1e-12
        assert np.max(np.abs(dv - rdv[keys])) <= 1e-12
        dk_sum += dk
        dv_sum += dv
    gq, gk, gv = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    assert np.max(np.abs(dk_sum - gk[0, keys, 0])) <= 1e-12
    assert np.max(np.abs(dv_sum - gv[0, keys, 0])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_head_forward_backward_matches_autograd_and_batched_routines(causal):
    """The whole-head routine (the reference of the full-size whole-head GPU
    tests) against an independent torch float64 autograd, and against the
    batched forward/backward on the same head: all five outputs, with rows
    taken in chunks smaller than the head (three chunks and a ragged one)."""
    pytest.importorskip("torch")
    x = inputs.dense_inputs(1, 230, 2, 1, 32, seed=13, round_bf16=False)
    scale = 0.21
    o_b, lse_b = ora.attention_forward(x["q"], x["k"], x["v"], scale, causal)
    dq_b, dk_b, dv_b = ora.attention_backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    dk_sum = np.zeros((230, 32))
    dv_sum = np.zeros((230, 32))
    for h in range(2):
        args = (x["q"][0, :, h], x["k"][0, :, 0], x["v"][0, :, 0], x["do"][0, :, h])
        got = ora.head_forward_backward(*args, scale, causal, row_chunk=64)
        ref = _torch_reference(*(a.astype(np.float64) for a in args), scale, causal)
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
            assert a.shape == b.shape, name
            assert np.max(np.abs(a - b)) <= 1e-12, name
        o, lse, dq, dk, dv = got
        assert np.max(np.abs(o - o_b[0, :, h])) <= 1e-12
        assert np.max(np.abs(lse - lse_b[0, h])) <= 1e-12
        assert np.max(np.abs(dq - dq_b[0, :, h])) <= 1e-12
        dk_sum += dk
        dv_sum += dv
    # the two query heads share key/value head 0: their dK, dV sum to the group's
    assert np.max(np.abs(dk_sum - dk_b[0, :, 0])) <= 1e-12
    assert np.max(np.abs(dv_sum - dv_b[0, :, 0])) <= 1e-12
