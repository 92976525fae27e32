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
  * wide score ranges (tests of the conditional rescale): the dense draws
    with key j scaled by 1 + growth j / N before rounding (ramp_inputs); or
    queries 1 + N(0, noise^2), the first 64 keys N(0, noise^2) and every later
    key one constant level (plateau_inputs);
  * tensors too large to draw on the host in seconds (tests of sizes past
    4 GiB per tensor): torch's counter-based Philox generator on the device,
    seeded per tensor (device_normal_bf16), standard-normal float32 rounded
    to bf16 by torch (nearest, ties to even); the oracle side copies back the
    slices it needs;
  * fp8 scores: the dense draws above before bf16 rounding; Q and K are each
    quantised per tensor to OCP e4m3 ("fn": largest finite 448, no
    infinities) with descale = amax(|x|) / 448 in float32 and bytes
    e4m3(x / descale), rounded to nearest, ties to even; V is bf16-rounded.
    The attention inputs the bytes stand for are descale * e4m3 value; the
    packed variant quantises the packed draws the same way.
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


def device_normal_bf16(shape, seed: int, device: str = "cuda"):
    """A standard-normal tensor drawn on the device by torch's Philox
    generator seeded with `seed`, rounded to bf16 (nearest, ties to even)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)


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


def ramp_inputs(B: int, N: int, Hq: int, Hkv: int, d: int, seed: int = 0,
                growth: float = 8.0) -> dict:
    """The dense draws with key j multiplied by 1 + growth * j / N before the
    bf16 rounding: key magnitudes grow along the sequence."""
    x = dense_inputs(B, N, Hq, Hkv, d, seed=seed, round_bf16=False)
    ramp = (1.0 + growth * np.arange(N, dtype=np.float32) / N)[None, :, None, None]
    x["k"] = x["k"] * ramp
    return {n: bf16_round(a) for n, a in x.items()}


def plateau_inputs(N: int, Hq: int, Hkv: int, d: int, level: float, seed: int = 0,
                   noise: float = 0.01, first: int = 64) -> dict:
    """Dense inputs with B = 1: every query 1 + noise, the first `first` keys
    pure noise, every later key equal to `level` in all components; noise
    ~ N(0, noise^2); V and dO ~ N(0, 1).  Drawn in the order Q-noise,
    K-noise, V, dO from Generator(PCG64(seed)), then bf16-rounded."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = 1.0 + noise * g.standard_normal((1, N, Hq, d), dtype=np.float32)
    k = noise * g.standard_normal((1, N, Hkv, d), dtype=np.float32)
    k[:, first:] = np.float32(level)
    v = g.standard_normal((1, N, Hkv, d), dtype=np.float32)
    do = g.standard_normal((1, N, Hq, d), dtype=np.float32)
    return {"q": bf16_round(q), "k": bf16_round(k), "v": bf16_round(v), "do": bf16_round(do)}


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


def varlen_qk_inputs(lengths_q, lengths_k, Hq: int, Hkv: int, d: int, seed: int = 0,
                     round_bf16: bool = True) -> dict:
    """Packed Q, dO [Tq, Hq, d] and K, V [Tk, Hkv, d] ~ N(0, 1), bf16-rounded
    unless asked not to, plus cu_seqlens_q and cu_seqlens_k."""
    if len(lengths_q) != len(lengths_k):
        raise ValueError("one query length and one key length per sequence")
    tq, tk = int(np.sum(lengths_q)), int(np.sum(lengths_k))
    g = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, t, h in (("q", tq, Hq), ("k", tk, Hkv), ("v", tk, Hkv), ("do", tq, Hq)):
        a = g.standard_normal((t, h, d), dtype=np.float32)
        out[name] = bf16_round(a) if round_bf16 else a
    out["cu_seqlens_q"] = cu_seqlens(lengths_q)
    out["cu_seqlens_k"] = cu_seqlens(lengths_k)
    return out


# ---------------------------------------------------------------------------
# OCP 8-bit floating point, e4m3 "fn" variant: 1 sign bit, 4 exponent bits
# (bias 7), 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6;
# the all-ones pattern 0x7f / 0xff is NaN, so the largest finite value is
# 0x7e = 1.75 * 2^8 = 448 and there are no infinities.


def _e4m3_magnitudes() -> np.ndarray:
    """Magnitudes of codes 0..127 (code 127, NaN in the format, gets 480: the
    value its bits would have, used only as the rounding neighbour of 448)."""
    c = np.arange(128)
    e = c >> 3
    m = (c & 7).astype(np.float64)
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))


_E4M3_MAG = _e4m3_magnitudes()


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of e4m3 bytes (uint8); NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = _E4M3_MAG[c & 0x7F]
    v = np.where(c & 0x80, -v, v)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode(x) -> np.ndarray:
    """Round values to the nearest e4m3 byte, ties to the even code; a value
    that would round beyond 448 raises ValueError (the format has no
    infinities).  Returns uint8."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode takes finite values only")
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_E4M3_MAG, a, side="left"), 1, 127)
    lo = hi - 1
    dlo = a - _E4M3_MAG[lo]
    dhi = _E4M3_MAG[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    if np.any(code == 127) or np.any(a > _E4M3_MAG[127]):
        raise ValueError("value out of the e4m3 range (largest finite 448)")
    sign = np.signbit(x)  # values that round to zero keep their sign (-0 is 0x80)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize_e4m3(x) -> tuple[np.ndarray, float]:
    """Per-tensor e4m3 quantisation: (bytes, descale) with descale =
    float32(amax / 448) so that descale * e4m3_decode(bytes) approximates x."""
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    descale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    return e4m3_encode(x.astype(np.float64) / descale), descale


def fp8_dense_inputs(B: int, N: int, Hq: int, Hkv: int, d: int, seed: int = 0) -> dict:
    """Dense fp8-score inputs: q8, k8 (uint8 e4m3 bytes), their descale
    factors, V (bf16-rounded float32) and the attention inputs q, k the bytes
    stand for (float64: descale * decoded value)."""
    raw = dense_inputs(B, N, Hq, Hkv, d, seed, round_bf16=False)
    q8, qd = quantize_e4m3(raw["q"])
    k8, kd = quantize_e4m3(raw["k"])
    return {"q8": q8, "k8": k8, "q_descale": qd, "k_descale": kd,
            "q": qd * e4m3_decode(q8), "k": kd * e4m3_decode(k8),
            "v": bf16_round(raw["v"])}


def fp8_varlen_qk_inputs(lengths_q, lengths_k, Hq: int, Hkv: int, d: int, seed: int = 0) -> dict:
    """Packed fp8-score inputs with separate query and key lengths: the draws
    of varlen_qk_inputs before bf16 rounding, Q and K quantised per tensor as
    in fp8_dense_inputs, V bf16-rounded, plus the offsets."""
    raw = varlen_qk_inputs(lengths_q, lengths_k, Hq, Hkv, d, seed, round_bf16=False)
    q8, qd = quantize_e4m3(raw["q"])
    k8, kd = quantize_e4m3(raw["k"])
    return {"q8": q8, "k8": k8, "q_descale": qd, "k_descale": kd,
            "q": qd * e4m3_decode(q8), "k": kd * e4m3_decode(k8),
            "v": bf16_round(raw["v"]),
            "cu_seqlens_q": raw["cu_seqlens_q"], "cu_seqlens_k": raw["cu_seqlens_k"]}
