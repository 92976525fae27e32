"""The library's launches under HIP graph capture: the dense forward and the
deterministic backward (semaphore-ordered and fixed-point dQ, the latter with
its K/V scan kernels), and the forward entry point that allocates nothing, are
captured once and replayed several times, with eager work and
synchronisations between the replays.  Every replay must reproduce the eager
results bit for bit.  The library records no memset and no host
synchronisation into the stream: the backward preprocess kernel clears the
dQ accumulator, the ticket and the semaphores itself on every call, so each
replay starts from the same state."""

import numpy as np
import pytest

from exact_attention_80_amd import inputs

from gpu_helpers import say, scale_for, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa as fa_mod
    return fa_mod


def same(a, b) -> bool:
    import torch
    return a.shape == b.shape and bool(torch.equal(a, b))


def eager_noise(t):
    """Unrelated eager work on the default stream between two replays."""
    import torch
    y = (t.float() * 3.0).sum()
    torch.cuda.synchronize()
    return float(y)


@pytest.mark.parametrize("det", [1, 4], ids=["ordered", "fixed"])
def test_dense_forward_and_deterministic_backward_replay(fa, det):
    import torch
    B, N, Hq, Hkv, d = 2, 300, 4, 2, 128
    say(f"graph replay dense B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal, dQ mode {det}")
    x = inputs.dense_inputs(B, N, Hq, Hkv, d, seed=71)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v", "do")}
    sc = scale_for(d)
    o0, lse0 = fa.fwd(t["q"], t["k"], t["v"], causal=True, softmax_scale=sc)
    g0 = fa.bwd(t["q"], t["k"], t["v"], o0, lse0, t["do"], causal=True, softmax_scale=sc,
                deterministic=det)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=True, softmax_scale=sc)
            fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=True, softmax_scale=sc,
                   deterministic=det)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=True, softmax_scale=sc)
        dq, dk, dv = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=True,
                            softmax_scale=sc, deterministic=det)
    for rep in range(4):
        eager_noise(t["q"])
        for buf in (o, lse, dq, dk, dv):
            buf.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}")
        assert same(o, o0) and same(lse, lse0), f"replay {rep}: forward differs"
        assert same(dq, g0[0]) and same(dk, g0[1]) and same(dv, g0[2]), \
            f"replay {rep}: backward differs"


def test_no_allocation_forward_replay(fa):
    import torch
    lq, lk, Hq, Hkv, d = [1, 17, 0, 300, 1], [9000, 2049, 40, 700, 5000], 8, 2, 128
    say(f"graph replay no-allocation forward lq={lq} lk={lk}")
    x = inputs.varlen_qk_inputs(lq, lk, Hq, Hkv, d, seed=72)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v")}
    cq = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    ck = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    Tq = t["q"].shape[0]
    o = torch.empty_like(t["q"])
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device="cuda")
    # eager call first: it also looks up the scratch array's device address
    fa.varlen_qk_fwd_noalloc(t["q"], t["k"], t["v"], cq, ck, causal=True, out=(o, lse))
    torch.cuda.synchronize()
    o0, lse0 = o.clone(), lse.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.varlen_qk_fwd_noalloc(t["q"], t["k"], t["v"], cq, ck, causal=True, out=(o, lse))
    for rep in range(4):
        eager_noise(t["k"])
        o.zero_()
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}")
        assert same(o, o0) and same(lse, lse0), f"replay {rep} differs"
    assert np.isfinite(o0.float().cpu().numpy()).all()
