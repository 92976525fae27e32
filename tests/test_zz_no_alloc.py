"""The no-allocation entry point (fa_varlen_qk_fwd_noalloc), called through the
C ABI, against the workspace entry point it stands in for (fa_varlen_qk_fwd):
the same kernels on the same schedule, so O and LSE must agree bit for bit.
Two calls in a row share the library's scratch array; the second, smaller
one must not see anything the first left there.  A problem too large for the
scratch is rejected on the host before any launch."""

import ctypes

import numpy as np
import pytest

from exact_attention_80_amd import inputs

from gpu_helpers import say, scale_for, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa as _fa
    return _fa


def problem(lq, lk, Hq, Hkv, d, seed):
    import torch
    x = inputs.varlen_qk_inputs(lq, lk, Hq, Hkv, d, seed=seed)
    t = {n: to_dev(x[n]) for n in ("q", "k", "v")}
    t["cq"] = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    t["ck"] = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    return t


def noalloc_raw(fa, t, Hq, Hkv, d, causal, o, lse):
    """fa_varlen_qk_fwd_noalloc through ctypes, into caller-provided outputs."""
    import torch
    lib = fa.raw()
    Tq, Tk = t["q"].shape[0], t["k"].shape[0]
    nseq = t["cq"].numel() - 1
    return lib.fa_varlen_qk_fwd_noalloc(
        t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(), lse.data_ptr(),
        t["cq"].data_ptr(), t["ck"].data_ptr(), nseq, Tq, Tk, 0, 0, Hq, Hkv, d,
        ctypes.c_float(scale_for(d)), int(causal),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


CASES = [
    # (query lengths, key lengths, Hq, Hkv, d): decode steps whose single
    # queries are split over chunks of a long key range, a prefill chunk, an
    # empty sequence; then a smaller batch
    (([1, 17, 0, 300, 1], [9000, 2049, 40, 700, 5000], 8, 2, 128),
     ([1, 5], [3000, 64], 4, 2, 128)),
    (([3, 1, 129], [4100, 70, 2100], 4, 1, 64),
     ([1], [1], 2, 1, 64)),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pair", CASES, ids=["d128", "d64"])
def test_noalloc_matches_workspace_entry_point(fa, pair, causal):
    import torch
    for lq, lk, Hq, Hkv, d in pair:
        say(f"noalloc lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
        t = problem(lq, lk, Hq, Hkv, d, seed=sum(lk) % 97)
        o_ref, lse_ref = fa.varlen_qk_fwd(t["q"], t["k"], t["v"], t["cq"], t["ck"],
                                          causal=causal, softmax_scale=scale_for(d))
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        st = noalloc_raw(fa, t, Hq, Hkv, d, causal, o, lse)
        assert st == 0, fa.raw().fa_last_error()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
        # the binding's wrapper takes the same path
        o2, lse2 = fa.varlen_qk_fwd_noalloc(t["q"], t["k"], t["v"], t["cq"], t["ck"],
                                           causal=causal, softmax_scale=scale_for(d))
        assert torch.equal(o2.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse2.view(torch.int32), lse_ref.view(torch.int32))


def test_noalloc_rejects_problems_beyond_the_scratch(fa):
    """A workspace beyond the limit is refused before any launch (outputs untouched)."""
    import torch
    Hq, Hkv, d = 64, 8, 256
    nseq, Tq, Tk = 400, 400, 400 * 2048
    need = fa.raw().fa_varlen_qk_fwd_workspace_size(nseq, Tq, Tk, Hq, Hkv, d, 1)
    assert need > fa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((Tq, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((Tk, Hkv, d), dtype=torch.bfloat16, device="cuda")
    cq = torch.arange(nseq + 1, dtype=torch.int32, device="cuda")
    ck = torch.arange(0, Tk + 1, 2048, dtype=torch.int32, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((Hq, Tq), 7.0, device="cuda")
    t = {"q": q, "k": k, "v": k, "cq": cq, "ck": ck}
    st = noalloc_raw(fa, t, Hq, Hkv, d, True, o, lse)
    assert st == 3  # FA_ERR_WORKSPACE
    assert b"no-allocation limit" in fa.raw().fa_last_error()
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
