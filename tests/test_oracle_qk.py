"""Pins for the oracle's packed batches with separate query and key lengths
(decode-shaped batches, bottom-right causal alignment).

Each check ties the new routines to something fixed independently: the
already-pinned square oracle (a bottom-right-aligned problem is the suffix of
a square causal one), a brute-force softmax loop, an independent torch
float64 autograd implementation, and central finite differences.
"""

import math

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora


def _batch(lq, lk, hq=2, hkv=1, d=16, seed=0):
    x = inputs.varlen_qk_inputs(lq, lk, hq, hkv, d, seed=seed)
    return {n: (a.astype(np.float64) if a.dtype != np.int32 else a) for n, a in x.items()}


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_reduce_to_the_packed_routines(causal):
    lens = [5, 33, 1, 64]
    x = _batch(lens, lens, hq=4, hkv=2, seed=3)
    o, lse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"], x["cu_seqlens_k"],
                                   0.3, causal)
    o2, lse2 = ora.varlen_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"], 0.3, causal)
    assert np.max(np.abs(o - o2)) <= 1e-12 and np.max(np.abs(lse - lse2)) <= 1e-12
    g = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                               x["cu_seqlens_k"], 0.3, causal)
    g2 = ora.varlen_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"], 0.3, causal)
    for a, b in zip(g, g2):
        assert np.max(np.abs(a - b)) <= 1e-12


@pytest.mark.parametrize("lq,lk", [(1, 37), (5, 5), (17, 64), (40, 100)])
def test_bottom_right_is_the_suffix_of_square_causal(lq, lk):
    """Queries that are the last lq positions of an lk-token context: their
    outputs are the last rows of the square causal problem, and dK, dV equal
    the square problem's when the earlier queries carry no output gradient."""
    x = _batch([lq], [lk], hq=2, hkv=1, d=8, seed=lq + lk)
    rng = np.random.Generator(np.random.PCG64(7))
    pre = lk - lq
    qsq = np.concatenate([rng.standard_normal((pre, 2, 8)), x["q"]])[None]
    dosq = np.concatenate([np.zeros((pre, 2, 8)), x["do"]])[None]
    ksq, vsq = x["k"][None], x["v"][None]
    o_sq, lse_sq = ora.attention_forward(qsq, ksq, vsq, 0.5, True)
    dq_sq, dk_sq, dv_sq = ora.attention_backward(qsq, ksq, vsq, dosq, 0.5, True)
    o, lse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                   x["cu_seqlens_k"], 0.5, True)
    dq, dk, dv = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                                        x["cu_seqlens_k"], 0.5, True)
    assert np.max(np.abs(o - o_sq[0, pre:])) <= 1e-12
    assert np.max(np.abs(lse - lse_sq[0][:, pre:])) <= 1e-12
    assert np.max(np.abs(dq - dq_sq[0, pre:])) <= 1e-12
    assert np.max(np.abs(dk - dk_sq[0])) <= 1e-12
    assert np.max(np.abs(dv - dv_sq[0])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_decode_row_is_a_softmax_over_every_key(causal):
    """A single query sees every key under either mask: brute-force loop."""
    lk, d, scale = 23, 4, 0.7
    x = _batch([1], [lk], hq=1, hkv=1, d=d, seed=5)
    q, k, v = x["q"][0, 0], x["k"][:, 0], x["v"][:, 0]
    s = [scale * sum(q[c] * k[j, c] for c in range(d)) for j in range(lk)]
    m = max(s)
    w = [math.exp(t - m) for t in s]
    z = sum(w)
    o_ref = [sum(w[j] * v[j, c] for j in range(lk)) / z for c in range(d)]
    lse_ref = m + math.log(z)
    o, lse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                   x["cu_seqlens_k"], scale, causal)
    assert np.max(np.abs(o[0, 0] - np.array(o_ref))) <= 1e-12
    assert abs(lse[0, 0] - lse_ref) <= 1e-12


def test_more_queries_than_keys():
    """Causal with lq > lk: the first lq - lk queries see no key (O = 0,
    LSE = -inf, dQ = 0); the rest are the square causal problem on lk keys."""
    lq, lk = 30, 12
    x = _batch([lq], [lk], hq=2, hkv=2, d=8, seed=9)
    o, lse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                   x["cu_seqlens_k"], 0.4, True)
    dq, dk, dv = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                                        x["cu_seqlens_k"], 0.4, True)
    e = lq - lk
    assert np.all(o[:e] == 0.0) and np.all(np.isneginf(lse[:, :e])) and np.all(dq[:e] == 0.0)
    o_sq, lse_sq = ora.attention_forward(x["q"][None, e:], x["k"][None], x["v"][None], 0.4, True)
    g_sq = ora.attention_backward(x["q"][None, e:], x["k"][None], x["v"][None], x["do"][None, e:],
                                  0.4, True)
    assert np.max(np.abs(o[e:] - o_sq[0])) <= 1e-12
    assert np.max(np.abs(lse[:, e:] - lse_sq[0])) <= 1e-12
    assert np.max(np.abs(dq[e:] - g_sq[0][0])) <= 1e-12
    assert np.max(np.abs(dk - g_sq[1][0])) <= 1e-12
    assert np.max(np.abs(dv - g_sq[2][0])) <= 1e-12


def test_empty_sequences():
    """A sequence without keys gives O = 0, LSE = -inf, dQ = 0; one without
    queries leaves its keys' dK, dV at zero; neither disturbs its neighbours."""
    lq, lk = [3, 0, 7, 4], [3, 10, 0, 6]
    x = _batch(lq, lk, hq=2, hkv=1, d=8, seed=13)
    for causal in (False, True):
        o, lse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                       x["cu_seqlens_k"], 0.5, causal)
        dq, dk, dv = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                                            x["cu_seqlens_k"], 0.5, causal)
        assert np.all(o[3:10] == 0.0) and np.all(np.isneginf(lse[:, 3:10])) and np.all(dq[3:10] == 0.0)
        assert np.all(dk[3:13] == 0.0) and np.all(dv[3:13] == 0.0)
        sub = _batch([3, 4], [3, 6], hq=2, hkv=1, d=8, seed=13)
        for a, name in ((slice(0, 3), "first"), (slice(10, 14), "last")):
            assert np.all(np.isfinite(o[a])), name
        # the neighbours match the same sequences computed on their own
        for (qa, qe, ka, ke) in ((0, 3, 0, 3), (10, 14, 13, 19)):
            cq = np.array([0, qe - qa], np.int32)
            ck = np.array([0, ke - ka], np.int32)
            o1, lse1 = ora.varlen_qk_forward(x["q"][qa:qe], x["k"][ka:ke], x["v"][ka:ke], cq, ck,
                                             0.5, causal)
            assert np.max(np.abs(o[qa:qe] - o1)) <= 1e-12
            assert np.max(np.abs(lse[:, qa:qe] - lse1)) <= 1e-12
        del sub


def _torch_bottom_right(q, k, v, do, scale, causal):
    import torch
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=(n != "do"))
         for n, a in (("q", q), ("k", k), ("v", v), ("do", do))}
    s = scale * t["q"] @ t["k"].T
    lq, lk = q.shape[0], k.shape[0]
    if causal:
        keep = torch.ones(lq, lk, dtype=torch.bool).tril(diagonal=lk - lq)
        s = s.masked_fill(~keep, float("-inf"))
    lse = torch.logsumexp(s, dim=1)
    o = torch.softmax(s, dim=1) @ t["v"]
    (o * t["do"]).sum().backward()
    return (o.detach().numpy(), lse.detach().numpy(), t["q"].grad.numpy(),
            t["k"].grad.numpy(), t["v"].grad.numpy())


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_with_bottom_right_mask(causal):
    """Independent implementation: torch float64 with the mask built by
    torch's own tril at diagonal lk - lq, per head, GQA groups summed."""
    pytest.importorskip("torch")
    lq, lk = [1, 9, 20, 3], [17, 9, 45, 3]
    hq, hkv, d, scale = 4, 2, 8, 0.35
    x = _batch(lq, lk, hq=hq, hkv=hkv, d=d, seed=21)
    o, lse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                   x["cu_seqlens_k"], scale, causal)
    dq, dk, dv = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                                        x["cu_seqlens_k"], scale, causal)
    cq, ck = x["cu_seqlens_q"], x["cu_seqlens_k"]
    dk_ref = np.zeros_like(dk)
    dv_ref = np.zeros_like(dv)
    for s in range(len(lq)):
        qa, qe, ka, ke = cq[s], cq[s + 1], ck[s], ck[s + 1]
        for h in range(hq):
            g = h // (hq // hkv)
            r = _torch_bottom_right(x["q"][qa:qe, h], x["k"][ka:ke, g], x["v"][ka:ke, g],
                                    x["do"][qa:qe, h], scale, causal)
            assert np.max(np.abs(o[qa:qe, h] - r[0])) <= 1e-12
            assert np.max(np.abs(lse[h, qa:qe] - r[1])) <= 1e-12
            assert np.max(np.abs(dq[qa:qe, h] - r[2])) <= 1e-12
            dk_ref[ka:ke, g] += r[3]
            dv_ref[ka:ke, g] += r[4]
    assert np.max(np.abs(dk - dk_ref)) <= 1e-12
    assert np.max(np.abs(dv - dv_ref)) <= 1e-12


def test_gradients_match_central_differences():
    """f = <O, dO> over a batch with lq < lk, lq > lk (empty rows) and lq = 1."""
    lq, lk = [4, 9, 1], [11, 5, 6]
    x = _batch(lq, lk, hq=2, hkv=1, d=4, seed=31)
    args = (x["cu_seqlens_q"], x["cu_seqlens_k"], 0.6, True)

    def f(q, k, v):
        o, _ = ora.varlen_qk_forward(q, k, v, *args)
        return float(np.sum(o * x["do"]))

    dq, dk, dv = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], *args)
    grads = {"q": dq, "k": dk, "v": dv}
    rng = np.random.Generator(np.random.PCG64(4))
    h = 1e-5
    for name in ("q", "k", "v"):
        for _ in range(12):
            u = rng.standard_normal(x[name].shape)
            p = {n: x[n] for n in ("q", "k", "v")}
            m = dict(p)
            p[name] = x[name] + h * u
            m[name] = x[name] - h * u
            fd = (f(p["q"], p["k"], p["v"]) - f(m["q"], m["k"], m["v"])) / (2 * h)
            an = float(np.sum(grads[name] * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_sampled_rows_and_keys_with_offset():
    """The spot-check routines with a causal offset agree with the full
    separate-length oracle (the full-size GPU tests use them)."""
    lq, lk, d = 40, 130, 8
    x = _batch([lq], [lk], hq=3, hkv=1, d=d, seed=41)
    off = lk - lq
    o, lse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                   x["cu_seqlens_k"], 0.3, True)
    dq, dk, dv = ora.varlen_qk_backward(x["q"], x["k"], x["v"], x["do"], x["cu_seqlens_q"],
                                        x["cu_seqlens_k"], 0.3, True)
    rows = np.array([0, 5, 39])
    keys = np.array([0, 90, 91, 129])
    dk_s = np.zeros((keys.size, d))
    dv_s = np.zeros((keys.size, d))
    for h in range(3):
        ro, rl, _, rdq = ora.head_query_rows(x["q"][:, h], x["k"][:, 0], x["v"][:, 0],
                                             x["do"][:, h], 0.3, True, rows, offset=off)
        assert np.max(np.abs(ro - o[rows, h])) <= 1e-12
        assert np.max(np.abs(rl - lse[h, rows])) <= 1e-12
        assert np.max(np.abs(rdq - dq[rows, h])) <= 1e-12
        a, b = ora.head_key_rows(x["q"][:, h], x["k"][:, 0], x["v"][:, 0], x["do"][:, h], 0.3,
                                 True, keys, row_chunk=7, offset=off)
        dk_s += a
        dv_s += b
    assert np.max(np.abs(dk_s - dk[keys, 0])) <= 1e-12
    assert np.max(np.abs(dv_s - dv[keys, 0])) <= 1e-12


def test_flop_count():
    """Non-causal: 4 d lq lk per head; equal lengths non-causal give the dense
    convention; a decode row sees all lk keys under the causal mask too."""
    f, b = ora.varlen_qk_flops([0, 3, 10], [0, 5, 9], 2, 8, False)
    assert f == 4 * 2 * 8 * (3 * 5 + 7 * 4) and b == 2.5 * f
    f1, _ = ora.varlen_qk_flops([0, 1], [0, 100], 4, 16, True)
    assert f1 == 4 * 4 * 16 * 100
    fd, _ = ora.attention_flops(1, 64, 2, 8, False)
    fv, _ = ora.varlen_qk_flops([0, 64], [0, 64], 2, 8, False)
    assert fd == fv
