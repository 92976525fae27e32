"""GPU parity past 4 GiB per tensor: one causal problem whose Q, K, V, O, dO,
dQ, dK, dV each span more than 2^32 bytes, so every address the kernels form
for late tokens needs 64-bit arithmetic (tile copies, buffer ranges, atomic
dQ adds, dK/dV stores).

B = 1, N = 2^17 + 64 tokens (a ragged last tile), Hq = Hkv = 128, d = 128: a
token's row is 32 KiB, a tensor 4.3 GB.  The inputs are drawn on the device
(inputs.device_normal_bf16); the oracle gets the slices it needs.  Checked
against the fp64 oracle, as in the other full-size tests: sampled query rows
(the first and last 32 plus random ones) of the first and last head (O, LSE,
dQ), the dK, dV of the last 256 keys of those heads, and for both heads the
size-independent identities sum_j dV_j = sum_i dO_i and sum_j dK_j = 0; and
the same tensors as a packed batch of two sequences, checked the same way on
the second one.
"""

import numpy as np
import pytest

from exact_attention_80_amd import inputs
from oracle import attention as ora

from gpu_helpers import TOL_GRAD, TOL_LSE, max_abs, o_excess, rel_fro, say, scale_for

pytestmark = pytest.mark.gpu

B, N, H, D = 1, (1 << 17) + 64, 128, 128
KEYS = 256
TOL_SUM = 1e-2


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def problem():
    import torch
    assert torch.cuda.is_available()
    from exact_attention_80_amd import fa
    say(f"large B={B} N={N} H={H} d={D} causal: {B * N * H * D * 2 / 2**30:.2f} GiB per tensor")
    assert B * N * H * D * 2 > (1 << 32)
    t = {name: inputs.device_normal_bf16((B, N, H, D), seed=70 + i)
         for i, name in enumerate(("q", "k", "v", "do"))}
    sc = scale_for(D)
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=True, softmax_scale=sc)
    g = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=True, softmax_scale=sc)
    torch.cuda.synchronize()
    yield t, o, lse, g, sc
    del t, o, lse, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("h", [0, H - 1])
def test_rows_keys_and_identities_past_4gib(problem, h):
    t, o, lse, (dq, dk, dv), sc = problem
    rng = np.random.Generator(np.random.PCG64(71 + h))
    rows = np.unique(np.r_[np.arange(32), np.arange(N - 32, N), rng.integers(0, N, 32)])
    qh, kh, vh, doh = (host(t[n][0, :, h]) for n in ("q", "k", "v", "do"))
    ro, rlse, _, rdq = ora.head_query_rows(qh, kh, vh, doh, sc, True, rows)
    pv = ora.head_query_rows(qh, kh, np.abs(vh), doh, sc, True, rows)[0]
    errs = dict(o=o_excess(host(o[0, rows, h]), ro, pv, N), lse=max_abs(host(lse[0, h, rows]), rlse),
                dq=rel_fro(host(dq[0, rows, h]), rdq))
    # the last keys: only the last queries see them
    keys = np.arange(N - KEYS, N)
    rdk, rdv = ora.head_key_rows(qh, kh, vh, doh, sc, True, keys)
    errs["dk"] = rel_fro(host(dk[0, N - KEYS:, h]), rdk)
    errs["dv"] = rel_fro(host(dv[0, N - KEYS:, h]), rdv)
    # identities over every key of the head
    sum_dv, sum_do = host(dv[0, :, h]).sum(axis=0), doh.sum(axis=0)
    dkh = host(dk[0, :, h])
    errs["sum_dv"] = float(np.linalg.norm(sum_dv - sum_do) / np.linalg.norm(sum_do))
    errs["sum_dk"] = float(np.linalg.norm(dkh.sum(axis=0)) / np.linalg.norm(np.abs(dkh).sum(axis=0)))
    say(f"h={h} rows={rows.size} errors {errs}")
    assert errs["o"] <= 1.0 and errs["lse"] <= TOL_LSE and errs["dq"] <= TOL_GRAD
    assert errs["dk"] <= TOL_GRAD and errs["dv"] <= TOL_GRAD
    assert errs["sum_dv"] <= TOL_SUM and errs["sum_dk"] <= TOL_SUM


def test_packed_batch_past_4gib(problem):
    """The same tensors as a packed batch [T, H, d] of two sequences (1000 and
    N - 1000 tokens): the second sequence's late rows and last keys, which
    lie past 2^32 bytes, against the oracle on that sequence alone."""
    import torch
    from exact_attention_80_amd import fa
    t, _, _, _, sc = problem
    first = 1000
    cu = torch.tensor([0, first, N], dtype=torch.int32, device="cuda")
    pk = {n: t[n][0] for n in ("q", "k", "v", "do")}
    o, lse = fa.varlen_fwd(pk["q"], pk["k"], pk["v"], cu, causal=True, softmax_scale=sc)
    dq, dk, dv = fa.varlen_bwd(pk["q"], pk["k"], pk["v"], o, lse, pk["do"], cu, causal=True,
                               softmax_scale=sc)
    torch.cuda.synchronize()
    h = 77
    L = N - first
    rng = np.random.Generator(np.random.PCG64(72))
    rows = np.unique(np.r_[np.arange(L - 32, L), rng.integers(0, L, 32)])
    qh, kh, vh, doh = (host(pk[n][first:, h]) for n in ("q", "k", "v", "do"))
    ro, rlse, _, rdq = ora.head_query_rows(qh, kh, vh, doh, sc, True, rows)
    pv = ora.head_query_rows(qh, kh, np.abs(vh), doh, sc, True, rows)[0]
    keys = np.arange(L - KEYS, L)
    rdk, rdv = ora.head_key_rows(qh, kh, vh, doh, sc, True, keys)
    errs = dict(o=o_excess(host(o[first + rows, h]), ro, pv, L),
                lse=max_abs(host(lse[h, first + rows]), rlse),
                dq=rel_fro(host(dq[first + rows, h]), rdq),
                dk=rel_fro(host(dk[N - KEYS:, h]), rdk), dv=rel_fro(host(dv[N - KEYS:, h]), rdv))
    say(f"packed h={h} rows={rows.size} errors {errs}")
    assert errs["o"] <= 1.0 and errs["lse"] <= TOL_LSE and errs["dq"] <= TOL_GRAD
    assert errs["dk"] <= TOL_GRAD and errs["dv"] <= TOL_GRAD
