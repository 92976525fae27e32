"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no attention arithmetic: it draws standard-normal tensors in
a fixed order from a PCG64 generator, rounds them to bfloat16 (round to
nearest even) and builds the packed variable-length batch layout.  Both the
HIP path and the CPU oracle receive exactly these values (bf16 -> fp64 is
lossless), so they can be compared element by element.

Recipe:
  * dense: Generator(PCG64(seed)), draws in the order Q, K, V, dO, each
    standard_normal float32 in the library layout ([B,N,Hq,d] for Q/dO,
    [B,N,Hkv,d] for K/V), then rounded to bf16;
  * variable length: lengths from a separate Generator(PCG64(length_seed)),
    each l = floor(exp(U(ln lo, ln(hi+1)))) clipped to [lo, hi]; when fewer
    than lo tokens would remain the last length absorbs them (or leaves lo for
    one more sequence when the remainder exceeds hi), so every length is in
    [lo, hi] and they sum exactly to the token total;
  * separate query and key lengths (decode-shaped batches): key lengths as
    above; then, from Generator(PCG64(query_seed)), per sequence in order a
    uniform draw u: u < decode_frac gives one query (a decode step), else the
    query count is an integer drawn uniformly from [1, min(Lk, qmax)] (a
    chunk of new tokens); Q, dO are [Tq, Hq, d] and K, V [Tk, Hkv, d], drawn
    in the order Q, K, V, dO.
"""

from __future__ import annotations

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = r.astype(np.uint32).view(np.float32).copy()
    out[nan] = np.nan
    return out


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable; call bf16_round first")
    return (u >> 16).astype(np.uint16)


def bits_to_f32(bits) -> np.ndarray:
    """float32 values of bf16 bit patterns (uint16 or int16)."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32)
    return (b << 16).view(np.float32)


def dense_inputs(B: int, N: int, Hq: int, Hkv: int, d: int, seed: int = 0,
                 round_bf16: bool = True) -> dict:
    """Q, K, V, dO ~ N(0, 1) in the dense layout; bf16-rounded unless asked not to."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, h in (("q", Hq), ("k", Hkv), ("v", Hkv), ("do", Hq)):
        a = g.standard_normal((B, N, h, d), dtype=np.float32)
        out[name] = bf16_round(a) if round_bf16 else a
    return out


def varlen_lengths(total: int = 65536, lo: int = 128, hi: int = 16384, seed: int = 1) -> list[int]:
    """Log-uniform sequence lengths in [lo, hi] that sum exactly to ``total``."""
    if total < lo:
        raise ValueError("total must be at least lo")
    g = np.random.Generator(np.random.PCG64(seed))
    lengths: list[int] = []
    rem = total
    while rem > 0:
        l = int(np.floor(np.exp(g.uniform(np.log(lo), np.log(hi + 1)))))
        l = min(max(l, lo), hi)
        if rem - l < lo:
            l = rem if rem <= hi else rem - lo
        lengths.append(l)
        rem -= l
    return lengths


def cu_seqlens(lengths) -> np.ndarray:
    """int32 prefix offsets [0, l0, l0+l1, ...] of the packed batch (drawn order)."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def varlen_inputs(lengths, Hq: int, Hkv: int, d: int, seed: int = 0) -> dict:
    """Packed Q, K, V, dO ~ N(0, 1) of shape [T, H, d], bf16-rounded, plus cu_seqlens."""
    T = int(np.sum(lengths))
    g = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, h in (("q", Hq), ("k", Hkv), ("v", Hkv), ("do", Hq)):
        out[name] = bf16_round(g.standard_normal((T, h, d), dtype=np.float32))
    out["cu_seqlens"] = cu_seqlens(lengths)
    return out


def qk_lengths(total_k: int = 65536, lo: int = 128, hi: int = 16384, seed: int = 2,
               query_seed: int = 3, decode_frac: float = 0.5, qmax: int = 1024):
    """(query lengths, key lengths) of a decode-shaped packed batch."""
    lk = varlen_lengths(total_k, lo, hi, seed)
    g = np.random.Generator(np.random.PCG64(query_seed))
    lq = []
    for k in lk:
        u = g.uniform()
        if u < decode_frac:
            lq.append(1)
        else:
            lq.append(int(g.integers(1, min(k, qmax) + 1)))
    return lq, lk


def varlen_qk_inputs(lengths_q, lengths_k, Hq: int, Hkv: int, d: int, seed: int = 0) -> dict:
    """Packed Q, dO [Tq, Hq, d] and K, V [Tk, Hkv, d] ~ N(0, 1), bf16-rounded,
    plus cu_seqlens_q and cu_seqlens_k."""
    if len(lengths_q) != len(lengths_k):
        raise ValueError("one query length and one key length per sequence")
    tq, tk = int(np.sum(lengths_q)), int(np.sum(lengths_k))
    g = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, t, h in (("q", tq, Hq), ("k", tk, Hkv), ("v", tk, Hkv), ("do", tq, Hq)):
        out[name] = bf16_round(g.standard_normal((t, h, d), dtype=np.float32))
    out["cu_seqlens_q"] = cu_seqlens(lengths_q)
    out["cu_seqlens_k"] = cu_seqlens(lengths_k)
    return out
