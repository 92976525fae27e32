"""Plain CPU oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module:
only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code, constants or helpers with the HIP kernels.

Everything is computed in float64 with NumPy, materialising the full score
matrix S and the probability matrix P for each head, exactly as standard
attention is defined; there is no online softmax, no tiling of the key axis
and no reordering.  The only concession to memory is that query rows are
processed in chunks of whole rows (every chunk still sees all keys of its
rows), which leaves each row's softmax the textbook one.

Sources (cited by page title and section):
  [FA2] "FlashAttention-2: Faster Attention with Better Parallelism and Work
        Partitioning (ICLR 2024)", wiki summary, sections "Problem and
        motivation" (standard attention materialises S = QK^T and
        P = softmax(S)) and "Core method" items 1 (only the logsumexp
        L = m + log(l) is kept for the backward), 2 (causal mask: keys with a
        column index above the row index are excluded) and 4 (MQA/GQA: K/V
        heads are shared by index mapping; the backward sums dK, dV over the
        implicitly replicated heads).
  [FA4B] "FlashAttention-4 backward: 2-CTA mode and performance" (CSDN
        blog), section 3.3.2: variable-length batches such as decode
        workloads, scheduled by per-tile cost.
  The backward formulas (recompute P from the logsumexp, dV = P^T dO,
  dP = dO V^T, dS = P o (dP - D) with D = rowsum(dO o O), dK = dS^T Q,
  dQ = dS K) are the chain rule of the forward definition.  Readings taken
  where the pages are silent:
    * dS is the gradient with respect to the *scaled* scores s = scale*q.k,
      so dQ = scale * dS K and dK = scale * dS^T Q (the true gradient; pinned
      by finite differences in the tests).
    * the logsumexp is the natural log of sum_j exp(scale * q_i . k_j).
    * causal masking is top-left aligned when queries and keys have the same
      length: key j is visible to query i iff j <= i.
    * packed batches whose sequences have different query and key lengths
      (Lq queries against Lk keys, the decode-shaped batches of [FA4B] 3.3.2)
      take the queries as the last Lq positions of the Lk-token context, so
      the causal mask is bottom-right aligned: key j is visible to query i
      iff j <= i + (Lk - Lq).
    * a query row that sees no key at all (causal with Lq > Lk, or Lk = 0)
      has an empty softmax: its output is 0, its logsumexp is ln 0 = -inf and
      it contributes nothing to any gradient.
    * GQA maps query head h to key/value head h // (Hq // Hkv).

Layouts (token-major, as in the library): dense Q/O/dO/dQ are [B, N, Hq, d],
K/V/dK/dV are [B, N, Hkv, d], the logsumexp is [B, Hq, N]; packed
variable-length tensors are [T, H, d] with cu_seqlens offsets and a
logsumexp of shape [Hq, T].
"""

from __future__ import annotations

import numpy as np

ROW_CHUNK = 2048


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _group(hq: int, hkv: int) -> int:
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"Hq={hq} must be a positive multiple of Hkv={hkv}")
    return hq // hkv


def head_scores(qh, kh, scale: float, causal: bool, row0: int = 0,
                offset: int = 0) -> np.ndarray:
    """Scaled score rows S[i, j] = scale * q_i . k_j for queries row0.. of one head.

    Causal: S[i, j] = -inf where key j > query i + offset ([FA2] "Core
    method" 2; offset = Lk - Lq aligns the mask bottom-right, 0 when the
    lengths are equal).
    """
    s = scale * (qh @ kh.T)
    if causal:
        rows = np.arange(row0, row0 + qh.shape[0])[:, None]
        cols = np.arange(kh.shape[0])[None, :]
        s = np.where(cols > rows + offset, -np.inf, s)
    return s


def head_probs(qh, kh, scale: float, causal: bool, row0: int = 0, offset: int = 0):
    """Row softmax of the scores and its natural-log normaliser.

    Returns (P, lse) with lse_i = ln sum_j exp(S_ij), computed stably as
    m_i + ln sum_j exp(S_ij - m_i), and P = exp(S - lse)
    ([FA2] "Problem and motivation"; "Core method" 1 for L = m + log l).
    A row with no visible key has lse = ln 0 = -inf and P = 0.
    """
    s = head_scores(qh, kh, scale, causal, row0, offset)
    if s.shape[1] == 0:
        return s.copy(), np.full(s.shape[0], -np.inf)
    m = s.max(axis=1)
    empty = m == -np.inf
    m_safe = np.where(empty, 0.0, m)
    with np.errstate(divide="ignore"):
        lse = m_safe + np.log(np.exp(s - m_safe[:, None]).sum(axis=1))
    lse = np.where(empty, -np.inf, lse)
    p = np.where(empty[:, None], 0.0, np.exp(s - np.where(empty, 0.0, lse)[:, None]))
    return p, lse


def attention_probs(q, k, scale: float, causal: bool) -> np.ndarray:
    """Full probability tensor P[b, h, i, j] (small inputs only; used by the pins)."""
    q, k = _f64(q), _f64(k)
    B, N, Hq, _ = q.shape
    G = _group(Hq, k.shape[2])
    out = np.empty((B, Hq, N, k.shape[1]))
    for b in range(B):
        for h in range(Hq):
            out[b, h], _ = head_probs(q[b, :, h], k[b, :, h // G], scale, causal)
    return out


def _head_forward(qh, kh, vh, scale, causal, row_chunk, offset=0):
    n = qh.shape[0]
    o = np.empty((n, vh.shape[1]))
    lse = np.empty(n)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        p, lse[r0:r1] = head_probs(qh[r0:r1], kh, scale, causal, r0, offset)
        o[r0:r1] = p @ vh
    return o, lse


def _head_backward(qh, kh, vh, doh, scale, causal, row_chunk, offset=0):
    """Gradients of one query head against its key/value head.

    Per chunk of whole query rows: recompute P from the definition, O = P V,
    D = rowsum(dO o O), dV += P^T dO, dP = dO V^T, dS = P o (dP - D),
    dQ = scale dS K, dK += scale dS^T Q.
    """
    n = qh.shape[0]
    dq = np.empty_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        q_c, do_c = qh[r0:r1], doh[r0:r1]
        p, _ = head_probs(q_c, kh, scale, causal, r0, offset)
        o_c = p @ vh
        d_c = (do_c * o_c).sum(axis=1)
        dv += p.T @ do_c
        dp = do_c @ vh.T
        ds = p * (dp - d_c[:, None])
        dq[r0:r1] = scale * (ds @ kh)
        dk += scale * (ds.T @ q_c)
    return dq, dk, dv


def attention_forward(q, k, v, scale: float, causal: bool, row_chunk: int = ROW_CHUNK):
    """Dense forward.  q [B,N,Hq,d], k/v [B,N,Hkv,d] -> (o [B,N,Hq,d], lse [B,Hq,N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, Hq, d = q.shape
    G = _group(Hq, k.shape[2])
    o = np.empty((B, N, Hq, v.shape[3]))
    lse = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            o[b, :, h], lse[b, h] = _head_forward(q[b, :, h], k[b, :, g], v[b, :, g],
                                                  scale, causal, row_chunk)
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool, row_chunk: int = ROW_CHUNK):
    """Dense backward -> (dq [B,N,Hq,d], dk [B,N,Hkv,d], dv [B,N,Hkv,d]).

    dK and dV of a key/value head are summed over the query heads of its group
    ([FA2] "Core method" 4).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    G = _group(Hq, Hkv)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            dqh, dkh, dvh = _head_backward(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h],
                                           scale, causal, row_chunk)
            dq[b, :, h] = dqh
            dk[b, :, g] += dkh
            dv[b, :, g] += dvh
    return dq, dk, dv


def _check_cu(cu, total):
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return cu


def varlen_forward(q, k, v, cu_seqlens, scale: float, causal: bool, row_chunk: int = ROW_CHUNK):
    """Packed variable-length forward: each sequence is attention on its own slice.

    q [T,Hq,d], k/v [T,Hkv,d] -> (o [T,Hq,d], lse [Hq,T]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = _check_cu(cu_seqlens, q.shape[0])
    o = np.zeros_like(q)
    lse = np.zeros((q.shape[1], q.shape[0]))
    for s in range(cu.size - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        o_s, lse_s = attention_forward(q[None, a:e], k[None, a:e], v[None, a:e],
                                       scale, causal, row_chunk)
        o[a:e] = o_s[0]
        lse[:, a:e] = lse_s[0]
    return o, lse


def varlen_backward(q, k, v, do, cu_seqlens, scale: float, causal: bool,
                    row_chunk: int = ROW_CHUNK):
    """Packed variable-length backward -> (dq [T,Hq,d], dk [T,Hkv,d], dv [T,Hkv,d])."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    cu = _check_cu(cu_seqlens, q.shape[0])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s in range(cu.size - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        g = attention_backward(q[None, a:e], k[None, a:e], v[None, a:e], do[None, a:e],
                               scale, causal, row_chunk)
        dq[a:e], dk[a:e], dv[a:e] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv


def _check_cu_pair(cu_q, cu_k, tq, tk):
    cu_q, cu_k = _check_cu(cu_q, tq), _check_cu(cu_k, tk)
    if cu_q.size != cu_k.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must describe the same number of sequences")
    return cu_q, cu_k


def varlen_qk_forward(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool,
                      row_chunk: int = ROW_CHUNK):
    """Packed forward with separate query and key lengths per sequence.

    Sequence s has queries cu_q[s]..cu_q[s+1] and keys cu_k[s]..cu_k[s+1];
    causal masking is bottom-right aligned (offset Lk - Lq), and rows that
    see no key give O = 0, LSE = -inf ([FA4B] 3.3.2 decode-shaped batches).
    q [Tq,Hq,d], k/v [Tk,Hkv,d] -> (o [Tq,Hq,d], lse [Hq,Tq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu_q, cu_k = _check_cu_pair(cu_seqlens_q, cu_seqlens_k, q.shape[0], k.shape[0])
    Hq = q.shape[1]
    G = _group(Hq, k.shape[1])
    o = np.zeros_like(q)
    lse = np.full((Hq, q.shape[0]), -np.inf)
    for s in range(cu_q.size - 1):
        qa, qe = int(cu_q[s]), int(cu_q[s + 1])
        ka, ke = int(cu_k[s]), int(cu_k[s + 1])
        if qe == qa:
            continue
        off = (ke - ka) - (qe - qa)
        for h in range(Hq):
            g = h // G
            o[qa:qe, h], lse[h, qa:qe] = _head_forward(q[qa:qe, h], k[ka:ke, g], v[ka:ke, g],
                                                       scale, causal, row_chunk, off)
    return o, lse


def varlen_qk_backward(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool,
                       row_chunk: int = ROW_CHUNK):
    """Packed backward with separate query and key lengths per sequence
    -> (dq [Tq,Hq,d], dk [Tk,Hkv,d], dv [Tk,Hkv,d]); dK, dV summed over the
    query heads of each group ([FA2] "Core method" 4)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    cu_q, cu_k = _check_cu_pair(cu_seqlens_q, cu_seqlens_k, q.shape[0], k.shape[0])
    Hq = q.shape[1]
    G = _group(Hq, k.shape[1])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s in range(cu_q.size - 1):
        qa, qe = int(cu_q[s]), int(cu_q[s + 1])
        ka, ke = int(cu_k[s]), int(cu_k[s + 1])
        if qe == qa or ke == ka:
            continue
        off = (ke - ka) - (qe - qa)
        for h in range(Hq):
            g = h // G
            dqh, dkh, dvh = _head_backward(q[qa:qe, h], k[ka:ke, g], v[ka:ke, g], do[qa:qe, h],
                                           scale, causal, row_chunk, off)
            dq[qa:qe, h] = dqh
            dk[ka:ke, g] += dkh
            dv[ka:ke, g] += dvh
    return dq, dk, dv


def varlen_qk_flops(cu_seqlens_q, cu_seqlens_k, Hq: int, d: int, causal: bool):
    """Algorithmic FLOPs of a packed batch with separate lengths: 4 d per
    visible (query, key) pair and query head for the forward (two products),
    2.5x that for the backward -- the dense convention counted exactly."""
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    pairs = 0
    for s in range(cu_q.size - 1):
        lq, lk = int(cu_q[s + 1] - cu_q[s]), int(cu_k[s + 1] - cu_k[s])
        if not causal:
            pairs += lq * lk
            continue
        i = np.arange(lq, dtype=np.int64)
        pairs += int(np.clip(i + (lk - lq) + 1, 0, lk).sum())
    f = 4.0 * Hq * d * pairs
    return f, 2.5 * f


def head_query_rows(qh, kh, vh, doh, scale: float, causal: bool, rows, offset: int = 0):
    """O, LSE, D and dQ of chosen query rows of one head, for spot checks at
    sizes where whole heads are too slow.

    A query row needs nothing but its own scores: S_i = scale q_i K^T (causal:
    keys j > i excluded), lse_i = m_i + ln sum_j exp(S_ij - m_i),
    P_i = exp(S_i - lse_i), O_i = P_i V, D_i = dO_i . O_i, dP_i = dO_i V^T,
    dS_i = P_i o (dP_i - D_i), dQ_i = scale dS_i K  ([FA2] "Problem and
    motivation", "Core method" 1-2; the backward is the chain rule).
    `offset` = Lk - Lq shifts the causal boundary (bottom-right alignment).
    Returns (o [r,d], lse [r], dvec [r], dq [r,d]) in the order of `rows`.
    """
    qh, kh, vh, doh = _f64(qh), _f64(kh), _f64(vh), _f64(doh)
    rows = np.asarray(rows, dtype=np.int64)
    s = scale * (qh[rows] @ kh.T)
    if causal:
        s = np.where(np.arange(kh.shape[0])[None, :] > rows[:, None] + offset, -np.inf, s)
    m = s.max(axis=1)
    empty = m == -np.inf
    m = np.where(empty, 0.0, m)
    with np.errstate(divide="ignore"):
        lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.where(empty[:, None], 0.0, np.exp(s - np.where(empty, 0.0, lse)[:, None]))
    lse = np.where(empty, -np.inf, lse)
    o = p @ vh
    do_r = doh[rows]
    dvec = (do_r * o).sum(axis=1)
    ds = p * (do_r @ vh.T - dvec[:, None])
    return o, lse, dvec, scale * (ds @ kh)


def head_key_rows(qh, kh, vh, doh, scale: float, causal: bool, keys,
                  row_chunk: int = ROW_CHUNK, offset: int = 0):
    """dK and dV that one query head contributes to chosen keys of its
    key/value head: dV_j = sum_i P_ij dO_i and dK_j = scale sum_i dS_ij q_i.

    Only queries that see a chosen key contribute (causal: i + offset >=
    min(keys), offset = Lk - Lq),
    but each of them needs its whole score row for its logsumexp and for
    D_i = dO_i . O_i; rows are taken in chunks of whole rows.  Summing the
    results over the query heads of a group gives the group's dK, dV
    ([FA2] "Core method" 4).  Returns (dk [r,d], dv [r,d]) in key order.
    """
    qh, kh, vh, doh = _f64(qh), _f64(kh), _f64(vh), _f64(doh)
    keys = np.asarray(keys, dtype=np.int64)
    n = qh.shape[0]
    dk = np.zeros((keys.size, kh.shape[1]))
    dv = np.zeros((keys.size, vh.shape[1]))
    first = max(0, int(keys.min()) - offset) if causal and keys.size else 0
    for r0 in range(first, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        q_c, do_c = qh[r0:r1], doh[r0:r1]
        p, _ = head_probs(q_c, kh, scale, causal, r0, offset)
        d_c = (do_c * (p @ vh)).sum(axis=1)
        p_k = p[:, keys]
        ds_k = p_k * (do_c @ vh[keys].T - d_c[:, None])
        dv += p_k.T @ do_c
        dk += scale * (ds_k.T @ q_c)
    return dk, dv


def head_forward_backward(qh, kh, vh, doh, scale: float, causal: bool,
                          row_chunk: int = ROW_CHUNK):
    """One query head end to end (used to time the oracle on a sample of heads).

    Returns (o, lse, dq, dk, dv) for that head.
    """
    qh, kh, vh, doh = _f64(qh), _f64(kh), _f64(vh), _f64(doh)
    o, lse = _head_forward(qh, kh, vh, scale, causal, row_chunk)
    dq, dk, dv = _head_backward(qh, kh, vh, doh, scale, causal, row_chunk)
    return o, lse, dq, dk, dv


def attention_flops(B: int, N: int, Hq: int, d: int, causal: bool) -> tuple[float, float]:
    """Algorithmic FLOP convention: forward 4 B Hq N^2 d (halved when causal),
    backward 2.5x the forward ([FA2] "Critical analysis": causal FLOPs halved)."""
    f = 4.0 * B * Hq * N * N * d * (0.5 if causal else 1.0)
    return f, 2.5 * f
