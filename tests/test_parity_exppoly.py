"""GPU parity of the forward builds whose exponentials are partly computed on
the FMA units ([FA4N] co-design list: a polynomial exponential beside the
hardware one): one probability in four (exppoly4) or in two (exppoly2) comes
from poly_exp2, whose relative error is at most 8.4e-5 plus a few fp32
roundings (pinned on the host, tests/test_exp2_poly.py).

A relative error eps in the probabilities moves O_id by at most
eps (sum_j P_ij |V_jd| + |O_id|) (numerator and row sum both move) and the LSE
by at most eps; the O bound therefore adds that term, and the LSE bar stays
1e-3.  Masked keys and rows that see no key must still give exact zeros."""

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora

from gpu_helpers import TOL_LSE, max_abs, o_excess, say, scale_for, to_dev, to_host

pytestmark = pytest.mark.gpu

EPS = 8.4e-5 + 6 * 2.0 ** -24


@pytest.fixture(scope="module", params=["exppoly4", "exppoly2"])
def lib(request):
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa
    return fa, fa.load_variant(request.param)


CASES = [
    # (B, N, Hq, Hkv, d): ragged tails, GQA, a single token, several tiles, d = 256
    (1, 200, 2, 2, 64),
    (2, 333, 4, 2, 128),
    (1, 1, 2, 1, 128),
    (1, 1000, 4, 4, 128),
    (1, 300, 2, 1, 256),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s)))
def test_poly_exp_forward_parity(lib, shape, causal):
    fa, L = lib
    B, N, Hq, Hkv, d = shape
    say(f"poly-exp fwd B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    x = inputs.dense_inputs(B, N, Hq, Hkv, d, seed=41)
    sc = scale_for(d)
    o, lse = fa.fwd(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), causal=causal,
                    softmax_scale=sc, lib=L)
    ro, rlse = ora.attention_forward(x["q"], x["k"], x["v"], sc, causal)
    pv, _ = ora.attention_forward(x["q"], x["k"], np.abs(x["v"]), sc, causal)
    o_h = to_host(o)
    errs = dict(o_excess=o_excess(o_h, ro, pv, N, extra=EPS * (pv + np.abs(ro))),
                lse=max_abs(to_host(lse), rlse))
    say(f"errors {errs}")
    assert errs["o_excess"] <= 1.0 and errs["lse"] <= TOL_LSE


def test_poly_exp_packed_rows_without_keys(lib):
    """Separate query and key lengths with empty sequences and more queries
    than keys: rows that see no key are exactly zero with LSE -inf."""
    import torch
    fa, L = lib
    lq, lk = [3, 0, 129, 40], [1, 50, 0, 700]
    say(f"poly-exp varlen_qk lq={lq} lk={lk}")
    x = inputs.varlen_qk_inputs(lq, lk, 4, 2, 128, seed=42)
    cq = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    ck = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    sc = scale_for(128)
    o, lse = fa.varlen_qk_fwd(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), cq, ck,
                              causal=True, softmax_scale=sc, lib=L)
    o, lse = to_host(o), to_host(lse)
    ro, rlse = ora.varlen_qk_forward(x["q"], x["k"], x["v"], x["cu_seqlens_q"],
                                     x["cu_seqlens_k"], sc, True)
    pv, _ = ora.varlen_qk_forward(x["q"], x["k"], np.abs(x["v"]), x["cu_seqlens_q"],
                                  x["cu_seqlens_k"], sc, True)
    empty = np.isneginf(rlse)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(o[empty.T] == 0.0)
    errs = dict(o_excess=o_excess(o, ro, pv, max(lk), extra=EPS * (pv + np.abs(ro))),
                lse=float(np.max(np.abs(lse[~empty] - rlse[~empty]))))
    say(f"errors {errs}")
    assert errs["o_excess"] <= 1.0 and errs["lse"] <= TOL_LSE
