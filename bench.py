"""Benchmark: causal self-attention forward + backward on one MI355X.

One step = one forward and one backward pass over one batch of the headline
workload (B=2, H=16, N=8192, d=128, bf16, causal), with seeded synthetic
inputs already resident in HBM.  The backward reduces dQ across key tiles with
fp32 atomic adds (--dq-mode 0, the default); --dq-mode 4 selects the int32
fixed-point adds, faster and bit-reproducible, whose resolution is set by a
per-head bound of the inputs (see include/fa.h).  Throughput counts the
algorithmic FLOPs 4*B*H*N^2*d/2 (forward) + 2.5x that (backward).

With --workload decode the step is instead one forward and one backward over
a packed batch whose sequences have separate query and key lengths (decode
steps and prefill chunks against their contexts), with FLOPs counted over the
(query, key) pairs the bottom-right causal mask leaves visible.

Prints one JSON line.  Besides the headline it carries:
  roofline      the dominant kernel (the backward main kernel): algorithmic
                FLOPs per launch / its average duration from HIP events recorded
                on its own stream during the timed steps, against the dense bf16
                MFMA peak; `traffic` is the kernel's HBM bytes per launch from
                the recorded rocprofv3 counter runs (profiles/), or null when
                the kernel sources changed since they were taken;
  extras        per-kernel times; in the atomic modes also the bytes of dQ
                atomic adds per backward launch and the rate they imply, to
                set beside what the atomics alone sustain (--atomic-probe):
                the dQ adds alone take most of that kernel's time (fp32) or
                well over half of it (int32), so they bound it together with
                its products;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample (whole query
                heads of the same workload) on this host's cores, scaled to the
                metric's unit.

Other modes: --sweep prints one line per measured workload (MHA 2K, the
headline, long context 16K/32K, GQA/MQA, the 65536-token packed batch; fast and
ordered and fixed-point dQ; with and without the longest-first tile order);
--atomic-probe measures the backward's fp32 and int32 dQ atomic adds alone
against plain stores of the same bytes; --device-info prints the CU count and clock; --workload decode times a
packed batch with separate query and key lengths.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 (256 CU x 4096 flop/clk x 2.4 GHz)
MFMA_FP8_PEAK_TFLOPS = 5033.2  # MI355X dense fp8 (twice the bf16 rate)
METRIC = "attention fwd+bwd TFLOPs/s (bf16, d=128, causal N=8K) and % of MFMA peak"


def flops(B, N, H, d, causal):
    f = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
    return f, 2.5 * f


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_main_traffic.txt")
# the backward's dQ reductions (the `deterministic` argument)
DQ_MODE_NAMES = ("atomic", "semaphore-ordered", "partial-tile", "fused partial-tile",
                 "fixed-point atomic")
KERNEL_SOURCES = ("fa_bwd.hip", "fa_common.h", "fa_launch.h")


def code_only(text: str) -> str:
    """C++ source without its comments and blank lines (so that editing a
    comment does not mark the recorded counters as stale)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash() -> str:
    """sha256 over the code (comments stripped) of the sources the backward
    main kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_80_amd", "csrc", name)) as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic(path: str, config: dict):
    """HBM bytes per launch of the backward main kernel from the recorded
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (each scaled by its copy-kernel
    calibration factor), or None when the record is missing, was taken on
    another workload, or the kernel sources changed since it was taken."""
    if not path or not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != kernel_source_hash() or rec.get("config") != config:
        return None
    return rec.get("bytes_per_launch")


def dq_reduction_bytes(B, N, Hq, d, causal):
    """fp32 bytes the backward main kernel adds into the dQ accumulator per launch:
    one 32-row x d tile per (query tile, key tile) pair the causal mask leaves
    visible, key tiles of 256 keys (128 for d = 256)."""
    bq, bc = 32, (128 if d == 256 else 256)
    nq, nkv = -(-N // bq), -(-N // bc)
    if causal:
        pairs = sum(min(nkv, (i * bq + bq - 1) // bc + 1) for i in range(nq))
    else:
        pairs = nq * nkv
    return pairs * B * Hq * bq * d * 4


def make_inputs(B, N, Hq, Hkv, d, seed=0):
    import numpy as np
    import torch

    from exact_attention_80_amd import inputs
    x = inputs.dense_inputs(B, N, Hq, Hkv, d, seed=seed)
    out = {}
    for n in ("q", "k", "v", "do"):
        bits = inputs.bf16_bits(x[n]).view(np.int16)
        out[n] = torch.from_numpy(np.ascontiguousarray(bits)).to("cuda").view(torch.bfloat16)
    return out


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity)."""
    return len(os.sched_getaffinity(0))


def blas_threads(n: int):
    """Context that runs the oracle's BLAS with n threads (threadpoolctl when
    present, else whatever the environment set)."""
    try:
        import threadpoolctl
        return threadpoolctl.threadpool_limits(limits=n)
    except Exception:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline(B, N, Hq, Hkv, d, causal, budget_s):
    """Oracle fwd+bwd on whole query heads of the workload's shape until
    budget_s elapses (at least one head), on every core of this process's
    affinity; the rate is scaled by the algorithmic FLOPs per head."""
    import numpy as np

    from exact_attention_80_amd import inputs
    from oracle import attention as ora
    cores = host_cores()
    scale = 1.0 / math.sqrt(d)
    g = np.random.Generator(np.random.PCG64(123))
    heads = 0
    with blas_threads(cores):
        t0 = time.perf_counter()
        while True:
            qh = inputs.bf16_round(g.standard_normal((N, d), dtype=np.float32))
            kh = inputs.bf16_round(g.standard_normal((N, d), dtype=np.float32))
            vh = inputs.bf16_round(g.standard_normal((N, d), dtype=np.float32))
            doh = inputs.bf16_round(g.standard_normal((N, d), dtype=np.float32))
            ora.head_forward_backward(qh, kh, vh, doh, scale, causal)
            heads += 1
            el = time.perf_counter() - t0
            if el >= budget_s or heads >= B * Hq:
                break
    f, b = flops(1, N, 1, d, causal)
    tflops = heads * (f + b) / el / 1e12
    return {
        "value": tflops, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"{heads} of {B * Hq} query heads (N={N}, d={d}, "
                  f"{'causal' if causal else 'non-causal'}) fwd+bwd in fp64, {el:.1f} s; "
                  f"rate scaled by algorithmic FLOPs per head",
    }


DECODE_METRIC = ("attention fwd+bwd TFLOPs/s (bf16, d=128, causal, packed batch with separate "
                 "query and key lengths) and % of MFMA peak")


def visible_pairs(lq, lk, causal):
    """(query, key) pairs a packed batch computes: Lq*Lk per sequence, or with
    the bottom-right causal mask sum_i clamp(i + Lk - Lq + 1, 0, Lk)."""
    total = 0
    for a, b in zip(lq, lk):
        if not causal:
            total += a * b
            continue
        off = b - a
        # rows i = 0..a-1 see min(b, max(0, i + off + 1)) keys
        for i in range(a):
            total += min(b, max(0, i + off + 1))
    return total


def decode_cpu_baseline(x, lq, lk, Hq, Hkv, d, budget_s):
    """Oracle fwd+bwd on whole (sequence, key/value head group) slices, in
    sequence order, until budget_s elapses; rate scaled by their FLOPs."""
    import numpy as np

    from oracle import attention as ora
    threads = host_cores()
    G = Hq // Hkv
    cq, ck = x["cu_seqlens_q"], x["cu_seqlens_k"]
    scale = 1.0 / math.sqrt(d)
    done_flops = 0.0
    units = 0
    limit = blas_threads(threads)
    limit.__enter__()
    t0 = time.perf_counter()
    for s in range(len(lq)):
        qa, qe, ka, ke = int(cq[s]), int(cq[s + 1]), int(ck[s]), int(ck[s + 1])
        one_q = np.array([0, qe - qa], np.int32)
        one_k = np.array([0, ke - ka], np.int32)
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            args = (x["q"][qa:qe, hs], x["k"][ka:ke, g:g + 1], x["v"][ka:ke, g:g + 1])
            ora.varlen_qk_forward(*args, one_q, one_k, scale, True)
            ora.varlen_qk_backward(*args, x["do"][qa:qe, hs], one_q, one_k, scale, True)
            done_flops += 3.5 * 4.0 * G * d * visible_pairs([qe - qa], [ke - ka], True)
            units += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    limit.__exit__(None, None, None)
    return {
        "value": done_flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{units} of {len(lq) * Hkv} (sequence, key/value head group) slices of the "
                  f"same batch, fwd+bwd in fp64, {el:.1f} s; rate scaled by their algorithmic FLOPs",
    }


def run_decode(args):
    """Packed batch with separate query and key lengths: 65536 keys in
    log-uniform sequences of 128..16384 tokens, half the sequences one query
    (a decode step), the rest a chunk of 1..1024 queries; Hq=32, Hkv=4, d=128,
    causal (bottom-right aligned)."""
    import numpy as np
    import torch

    from exact_attention_80_amd import fa, inputs

    Hq, Hkv, d = 32, 4, 128
    det = args.dq_mode
    if det in (2, 3):
        print("bench.py: the partial-tile dQ reductions are dense-only", file=sys.stderr)
        sys.exit(2)
    lq, lk = inputs.qk_lengths()
    x = inputs.varlen_qk_inputs(lq, lk, Hq, Hkv, d, seed=0)
    t = {}
    for n in ("q", "k", "v", "do"):
        bits = inputs.bf16_bits(x[n]).view(np.int16)
        t[n] = torch.from_numpy(np.ascontiguousarray(bits)).to("cuda").view(torch.bfloat16)
    cq = torch.from_numpy(x["cu_seqlens_q"]).to("cuda")
    ck = torch.from_numpy(x["cu_seqlens_k"]).to("cuda")
    Tq, Tk = sum(lq), sum(lk)
    scale = 1.0 / math.sqrt(d)
    wsf = fa.varlen_qk_fwd_workspace(len(lq), Tq, Tk, Hq, Hkv, d, True, "cuda")
    wsb = fa.varlen_qk_bwd_workspace(len(lq), Tq, Tk, Hq, Hkv, d, True, det, "cuda")

    def step():
        o, lse = fa.varlen_qk_fwd(t["q"], t["k"], t["v"], cq, ck, causal=True,
                                  softmax_scale=scale, workspace=wsf)
        fa.varlen_qk_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=True,
                         softmax_scale=scale, deterministic=det, workspace=wsb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fa.timing_begin()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kt = fa.timing_end()

    pairs = visible_pairs(lq, lk, True)
    f_fwd = 4.0 * Hq * d * pairs
    f_bwd = 2.5 * f_fwd
    value = (f_fwd + f_bwd) / (elapsed / args.steps) / 1e12
    ms = {k: kt[k][1] / max(1, kt[k][0]) for k in ("fwd", "bwd_main", "bwd_pre", "bwd_post", "sched")}
    # the dominant kernel of this workload
    dom = "bwd_main" if ms["bwd_main"] >= ms["fwd"] else "fwd"
    f_dom = f_bwd if dom == "bwd_main" else f_fwd
    achieved = f_dom / (ms[dom] * 1e-3) / 1e12
    # compulsory HBM bytes of the forward: Q, K, V read, O written (bf16), LSE (fp32)
    fwd_bytes = 2 * d * (2 * Tq * Hq + 2 * Tk * Hkv) + 4 * Tq * Hq
    extras = {
        "fwd_kernel_ms": ms["fwd"], "fwd_tflops": f_fwd / (ms["fwd"] * 1e-3) / 1e12,
        "fwd_compulsory_hbm_gbps": fwd_bytes / (ms["fwd"] * 1e-3) / 1e9,
        "bwd_main_kernel_ms": ms["bwd_main"], "bwd_pre_ms": ms["bwd_pre"],
        "bwd_post_ms": ms["bwd_post"], "sched_ms_per_call": ms["sched"],
        "bwd_tflops": f_bwd / (ms["bwd_main"] * 1e-3) / 1e12,
        "visible_pairs_per_head": pairs, "nseq": len(lq), "total_q": Tq, "total_k": Tk,
    }
    if args.extra and args.steps > 0:
        # the forward with fp8 (e4m3) Q and K for the scores, per-tensor descale factors
        qd = float(t["q"].float().abs().max()) / 448.0
        kd = float(t["k"].float().abs().max()) / 448.0
        q8 = (t["q"].float() / qd).to(torch.float8_e4m3fn)
        k8 = (t["k"].float() / kd).to(torch.float8_e4m3fn)
        for _ in range(3):
            fa.varlen_qk_fwd_fp8(q8, k8, t["v"], cq, ck, qd, kd, causal=True,
                                 softmax_scale=scale, workspace=wsf)
        torch.cuda.synchronize()
        fa.timing_begin()
        for _ in range(args.steps):
            fa.varlen_qk_fwd_fp8(q8, k8, t["v"], cq, ck, qd, kd, causal=True,
                                 softmax_scale=scale, workspace=wsf)
        kf = fa.timing_end()["fwd"]
        fp8_ms = kf[1] / max(1, kf[0])
        extras["fp8_fwd_kernel_ms"] = fp8_ms
        extras["fp8_fwd_tflops"] = f_fwd / (fp8_ms * 1e-3) / 1e12
        extras["fp8_fwd_speedup_vs_bf16"] = ms["fwd"] / fp8_ms
        del q8, k8
    line = {
        "metric": DECODE_METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"causal packed batch with separate query and key lengths: {len(lq)} "
                        f"sequences, {Tq} queries against {Tk} keys (half one-query decode steps), "
                        f"Hq={Hq} Hkv={Hkv} d={d}, "
                        f"{DQ_MODE_NAMES[det]} dQ reduction",
            "nseq": len(lq), "total_q": Tq, "total_k": Tk, "Hq": Hq, "Hkv": Hkv, "d": d,
            "causal": True, "deterministic": det,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": {"bwd_main": "bwd_kernel (backward main)", "fwd": "fwd_kernel"}[dom],
            "achieved": achieved,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
        },
        "extras": extras,
    }
    if args.cpu_budget > 0:
        line["cpu_baseline"] = decode_cpu_baseline(x, lq, lk, Hq, Hkv, d, args.cpu_budget)
    print(json.dumps(line), flush=True)


def measure_dense(fa, x, B, N, Hq, Hkv, d, causal, det, steps, warmup):
    """Time `steps` forward+backward steps on resident inputs; returns the wall
    time per step and the average of every kernel's HIP-event time (ms)."""
    import torch
    scale = 1.0 / math.sqrt(d)
    ws = fa.bwd_workspace(x["q"], x["k"], causal, det)

    def step():
        o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=causal, softmax_scale=scale)
        fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal, softmax_scale=scale,
               deterministic=det, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    fa.timing_begin()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kt = fa.timing_end()
    del ws
    avg = {k: v[1] / max(1, v[0]) for k, v in kt.items()}
    avg["bwd_total"] = sum(kt[k][1] for k in ("bwd_pre", "bwd_main", "bwd_post")) / max(
        1, kt["bwd_main"][0])
    return elapsed * 1e3 / steps, avg


def varlen_flops(lengths, Hq, d, causal):
    """The dense convention per sequence: 4 Hq L^2 d, halved when causal."""
    f = sum(4.0 * Hq * L * L * d * (0.5 if causal else 1.0) for L in lengths)
    return f, 2.5 * f


def varlen_cpu_baseline(x, lengths, Hq, Hkv, d, causal, budget_s):
    """Oracle fwd+bwd of whole sequences of the packed batch (all heads), in
    order until budget_s elapses; rate scaled by their algorithmic FLOPs."""
    import numpy as np

    from oracle import attention as ora
    cores = host_cores()
    cu = x["cu_seqlens"]
    scale = 1.0 / math.sqrt(d)
    done, n = 0.0, 0
    with blas_threads(cores):
        t0 = time.perf_counter()
        for s in range(len(lengths)):
            a, e = int(cu[s]), int(cu[s + 1])
            one = np.array([0, e - a], np.int32)
            sl = {k: x[k][a:e] for k in ("q", "k", "v", "do")}
            ora.varlen_forward(sl["q"], sl["k"], sl["v"], one, scale, causal)
            ora.varlen_backward(sl["q"], sl["k"], sl["v"], sl["do"], one, scale, causal)
            f, b = varlen_flops([e - a], Hq, d, causal)
            done += f + b
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
    return {"value": done / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {len(lengths)} sequences (all {Hq} heads) fwd+bwd in fp64, "
                      f"{el:.1f} s; rate scaled by their algorithmic FLOPs"}


def measure_varlen(fa, t, cu, lengths, Hq, Hkv, d, causal, det, steps, warmup):
    import torch
    T = sum(lengths)
    scale = 1.0 / math.sqrt(d)
    wsf = fa.varlen_fwd_workspace(len(lengths), T, Hq, Hkv, d, causal, "cuda")
    wsb = fa.varlen_bwd_workspace(len(lengths), T, Hq, Hkv, d, causal, det, "cuda")

    def step():
        o, lse = fa.varlen_fwd(t["q"], t["k"], t["v"], cu, causal=causal, softmax_scale=scale,
                               max_seqlen=max(lengths), workspace=wsf)
        fa.varlen_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cu, causal=causal,
                      softmax_scale=scale, deterministic=det, max_seqlen=max(lengths),
                      workspace=wsb)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    fa.timing_begin()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kt = fa.timing_end()
    if det:
        assert fa.workspace_error(wsb) == 0
    avg = {k: v[1] / max(1, v[0]) for k, v in kt.items()}
    avg["bwd_total"] = sum(kt[k][1] for k in ("bwd_pre", "bwd_main", "bwd_post", "sched")) / max(
        1, kt["bwd_main"][0])
    avg["fwd_total"] = sum(kt[k][1] for k in ("fwd", "fwd_combine")) / max(1, kt["fwd"][0]) + \
        avg["sched"]
    return elapsed * 1e3 / steps, avg


SWEEP_DENSE = [
    # (config id, B, N, Hq, Hkv, d, causal)
    ("C1", 4, 2048, 16, 16, 64, False), ("C1", 4, 2048, 16, 16, 64, True),
    ("C1", 4, 2048, 16, 16, 128, False), ("C1", 4, 2048, 16, 16, 128, True),
    ("H", 2, 8192, 16, 16, 128, True),
    ("C2", 1, 16384, 16, 16, 128, True), ("C2", 1, 32768, 16, 16, 128, True),
    ("C3", 2, 8192, 32, 4, 128, True), ("C3", 2, 8192, 32, 1, 128, True),
]


def sweep_line(cid, workload, value_flops, ms_step, avg, f_fwd, f_bwd, det, sched, cpu, extra):
    fwd_ms = avg.get("fwd_total", avg["fwd"])
    line = {
        "sweep": cid, "workload": workload,
        "dq_reduction": DQ_MODE_NAMES[det],
        "tile_order": sched,
        "value": value_flops / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s",
        "pct_of_peak": 100.0 * value_flops / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "ms_per_step": ms_step,
        "fwd_ms": fwd_ms, "fwd_tflops": f_fwd / (fwd_ms * 1e-3) / 1e12,
        "fwd_pct_peak": 100.0 * f_fwd / (fwd_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "bwd_ms": avg["bwd_total"], "bwd_main_ms": avg["bwd_main"],
        "bwd_tflops": f_bwd / (avg["bwd_total"] * 1e-3) / 1e12,
        "bwd_pct_peak": 100.0 * f_bwd / (avg["bwd_total"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "cpu_baseline": cpu,
    }
    line.update(extra)
    return line


def run_sweep(args):
    """One JSON line per workload of the scope table's measurement row: MHA 2K
    (d = 64, 128; causal and not), the headline, long context 16K / 32K, GQA
    / MQA, and the 65536-token packed batch; each with fp32 atomic,
    semaphore-ordered and fixed-point dQ, plus the headline and the packed
    batch with the longest-first tile order switched off (FA_SCHED=natural)."""
    import torch

    from exact_attention_80_amd import fa, inputs
    torch.cuda.set_device(0)
    cpu_cache = {}
    want = set(args.sweep_ids.split(",")) if args.sweep_ids else None
    for cid, B, N, Hq, Hkv, d, causal in SWEEP_DENSE:
        if want is not None and cid not in want:
            continue
        x = make_inputs(B, N, Hq, Hkv, d)
        f_fwd, f_bwd = flops(B, N, Hq, d, causal)
        key = (N, d, causal)
        if key not in cpu_cache:
            cpu_cache[key] = (cpu_baseline(B, N, Hq, Hkv, d, causal, args.cpu_budget)
                              if args.cpu_budget > 0 else None)
        scheds = ("longest-first", "natural") if cid == "H" else ("longest-first",)
        # one discarded run first, so that the first timed row is as warm as
        # the others (clocks, first touch of the new buffers)
        measure_dense(fa, x, B, N, Hq, Hkv, d, causal, 0, max(10, args.steps), args.warmup)
        for det in (0, 1, 4):
            for sched in scheds:
                if sched == "natural":
                    os.environ["FA_SCHED"] = "natural"
                try:
                    ms, avg = measure_dense(fa, x, B, N, Hq, Hkv, d, causal, det, args.steps,
                                            args.warmup)
                finally:
                    os.environ.pop("FA_SCHED", None)
                wl = (f"{'causal' if causal else 'non-causal'} B={B} Hq={Hq} Hkv={Hkv} N={N} "
                      f"d={d}")
                print(json.dumps(sweep_line(cid, wl, f_fwd + f_bwd, ms, avg, f_fwd, f_bwd, det,
                                            sched, cpu_cache[key], {})), flush=True)
        del x
        torch.cuda.empty_cache()
    # C4: the packed batch
    if want is not None and "C4" not in want:
        return
    lengths = inputs.varlen_lengths()
    Hq = Hkv = 16
    d = 128
    xv = inputs.varlen_inputs(lengths, Hq, Hkv, d, seed=4)
    t = {}
    for n in ("q", "k", "v", "do"):
        bits = inputs.bf16_bits(xv[n]).view("int16")
        t[n] = torch.from_numpy(bits.copy()).to("cuda").view(torch.bfloat16)
    cu = torch.from_numpy(xv["cu_seqlens"]).to("cuda")
    f_fwd, f_bwd = varlen_flops(lengths, Hq, d, True)
    cpu = (varlen_cpu_baseline(xv, lengths, Hq, Hkv, d, True, args.cpu_budget)
           if args.cpu_budget > 0 else None)
    measure_varlen(fa, t, cu, lengths, Hq, Hkv, d, True, 0, max(10, args.steps),
                   args.warmup)  # discarded, as for the dense workloads
    for det in (0, 1, 4):
        for sched in ("longest-first", "natural"):
            if sched == "natural":
                os.environ["FA_SCHED"] = "natural"
            try:
                ms, avg = measure_varlen(fa, t, cu, lengths, Hq, Hkv, d, True, det, args.steps,
                                         args.warmup)
            finally:
                os.environ.pop("FA_SCHED", None)
            wl = (f"causal packed batch of {len(lengths)} sequences, {sum(lengths)} tokens "
                  f"(log-uniform lengths 128..16384, longest {max(lengths)}), Hq=Hkv={Hq} d={d}")
            print(json.dumps(sweep_line("C4", wl, f_fwd + f_bwd, ms, avg, f_fwd, f_bwd, det, sched,
                                        cpu, {"lengths": lengths})), flush=True)


def run_atomic_probe(args):
    """What the backward's dQ reductions can sustain: its fp32 atomic adds
    alone (same instructions, same 32 x 16 per-wave blocks of a [rows, Hq*d]
    fp32 accumulator, 1024 workgroups), the fixed-point mode's int32 atomic
    adds in the same pattern, and plain stores of the same bytes; the
    headline backward moves 2.21 GB this way per launch."""
    import torch

    from exact_attention_80_amd import fa
    torch.cuda.set_device(0)
    rows, row_floats = 2 * 8192, 16 * 128          # the headline's dQ accumulator
    blocks, items = 1024, 132                     # 1024 x 132 x 16 KiB = 2.21 GB
    out = {"probe": "dq_reduction", "rows": rows, "row_floats": row_floats,
           "blocks": blocks, "items": items}
    for kind, key in ((0, "atomic"), (2, "int_atomic"), (1, "store")):
        buf = torch.zeros((rows, row_floats), dtype=torch.float32, device="cuda")
        launches = 0
        for _ in range(2):
            fa.probe_dq_reduction(buf, blocks, items, kind)
        launches += 2
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        reps = 10
        nbytes = 0
        for _ in range(reps):
            nbytes += fa.probe_dq_reduction(buf, blocks, items, kind)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        launches += reps
        out[f"{key}_ms"] = ms
        out[f"{key}_tbps"] = nbytes / reps / (ms * 1e-3) / 1e12
        out["bytes_per_launch"] = nbytes // reps
        if kind != 1:
            # every atomic launch added 1/1024 (fp32) or 1 (int32) to each
            # element of the 4096-element tiles it visited, exactly: all adds landed
            per = 1.0 / 1024 if kind == 0 else 1.0
            want = launches * blocks * items * 4096 * per
            got = float((buf if kind == 0 else buf.view(torch.int32)).double().sum())
            out[f"{key}_sum_check"] = got == want
            if got != want:
                raise RuntimeError(f"probe sum {got} != {want} ({key})")
        del buf
    print(json.dumps(out), flush=True)


def device_info():
    """CU count and clocks of the device (rocminfo), for the record."""
    import subprocess
    info = {}
    try:
        r = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60)
        agent = None
        for line in r.stdout.splitlines():
            line = line.strip()
            if line.startswith("Name:") and "gfx" in line:
                agent = line.split(":", 1)[1].strip()
                info["name"] = agent
            if agent and line.startswith("Compute Unit:"):
                info["compute_units"] = int(line.split(":", 1)[1])
            if agent and line.startswith("Max Clock Freq. (MHz):"):
                info["max_clock_mhz"] = int(line.split(":", 1)[1])
            if agent and "compute_units" in info and "max_clock_mhz" in info:
                break
    except Exception as e:  # pragma: no cover
        info["error"] = str(e)
    return info


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="headline", choices=("headline", "decode"),
                    help="headline: causal B=2 H=16 N=8192 d=128; decode: packed batch with "
                         "separate query and key lengths (Hq=32, Hkv=4, d=128)")
    ap.add_argument("--steps", type=int, default=30)
    # the first ten or so steps of a process run slower while the clocks settle
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--B", type=int, default=2)
    ap.add_argument("--N", type=int, default=8192)
    ap.add_argument("--H", type=int, default=16)
    ap.add_argument("--Hkv", type=int, default=0)
    ap.add_argument("--d", type=int, default=128)
    ap.add_argument("--non-causal", action="store_true")
    ap.add_argument("--dq-mode", type=int, default=0, choices=(0, 1, 2, 3, 4),
                    help="dQ reduction: 0 fp32 atomics, 1 semaphore-ordered, 2 partial tiles "
                         "summed by a second kernel, 3 partial tiles summed by the last "
                         "contributor, 4 int32 fixed-point atomics")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 disables it)")
    ap.add_argument("--traffic-file", default=TRAFFIC_FILE,
                    help="recorded HBM bytes per launch of the dominant kernel")
    ap.add_argument("--extra", action="store_true",
                    help="also time the backward with the other dQ reduction modes and the "
                         "forward with fp8 scores (extras)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--variants", action="store_true",
                    help="also time the forward of every build variant beside the library "
                         "(extras fwd_<variant>_kernel_ms)")
    ap.add_argument("--sweep", action="store_true",
                    help="one JSON line per measured workload (MHA 2K, headline, 16K/32K, "
                         "GQA/MQA, packed batch; fp32 atomic, ordered and fixed-point dQ; "
                         "tile-order ablation)")
    ap.add_argument("--sweep-ids", default="",
                    help="with --sweep: only these workload ids, comma-separated "
                         "(C1, H, C2, C3, C4)")
    ap.add_argument("--atomic-probe", action="store_true",
                    help="only measure the rate of the backward's dQ atomics and of plain "
                         "stores of the same bytes")
    ap.add_argument("--device-info", action="store_true",
                    help="only print the device's CU count and clock (rocminfo)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding across GPUs is not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy_mib > 0:
        # a plain copy of known size: reads and writes calibrate FETCH_SIZE / WRITE_SIZE
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "read_bytes": n, "write_bytes": n}), flush=True)
        return

    if args.device_info:
        print(json.dumps(device_info()), flush=True)
        return
    if args.atomic_probe:
        run_atomic_probe(args)
        return
    if args.sweep:
        run_sweep(args)
        return

    if args.workload == "decode":
        torch.cuda.set_device(0)
        run_decode(args)
        return

    from exact_attention_80_amd import fa

    B, N, Hq, d = args.B, args.N, args.H, args.d
    Hkv = args.Hkv or Hq
    causal = not args.non_causal
    det = args.dq_mode
    scale = 1.0 / math.sqrt(d)
    torch.cuda.set_device(0)
    x = make_inputs(B, N, Hq, Hkv, d)
    ws = fa.bwd_workspace(x["q"], x["k"], causal, det)

    def step():
        o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=causal, softmax_scale=scale)
        fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal, softmax_scale=scale,
               deterministic=det, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fa.timing_begin()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kt = fa.timing_end()

    f_fwd, f_bwd = flops(B, N, Hq, d, causal)
    ms_step = elapsed * 1e3 / args.steps
    value = (f_fwd + f_bwd) / (elapsed / args.steps) / 1e12

    n_fwd, ms_fwd = kt["fwd"]
    n_bwd, ms_bwd = kt["bwd_main"]
    n_pre, ms_pre = kt["bwd_pre"]
    n_post, ms_post = kt["bwd_post"]
    avg_bwd_ms = ms_bwd / max(1, n_bwd)
    avg_fwd_ms = ms_fwd / max(1, n_fwd)
    achieved = f_bwd / (avg_bwd_ms * 1e-3) / 1e12
    traffic = measured_traffic(args.traffic_file,
                               {"B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d, "causal": causal,
                                "deterministic": det})

    extras = {
        "fwd_kernel_ms": avg_fwd_ms,
        "fwd_tflops": f_fwd / (avg_fwd_ms * 1e-3) / 1e12,
        "fwd_pct_peak": 100.0 * f_fwd / (avg_fwd_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "bwd_main_kernel_ms": avg_bwd_ms,
        "bwd_pre_ms": ms_pre / max(1, n_pre),
        "bwd_post_ms": ms_post / max(1, n_post),
        "bwd_tflops": f_bwd / ((ms_bwd + ms_pre + ms_post) / max(1, n_bwd) * 1e-3) / 1e12,
        "pct_of_peak": 100.0 * value / MFMA_BF16_PEAK_TFLOPS,
    }
    if det in (0, 4):
        # the atomic modes' dQ reduction: device-scope fp32 (int32) atomic adds; the
        # rate they imply over the kernel's time, against what they sustain
        # alone (--atomic-probe), shows how close the kernel is to that bound
        dq_bytes = dq_reduction_bytes(B, N, Hq, d, causal)
        extras["bwd_dq_atomic_bytes"] = dq_bytes
        extras["bwd_dq_atomic_tbps"] = dq_bytes / (avg_bwd_ms * 1e-3) / 1e12
    if args.extra:
        o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=causal, softmax_scale=scale)
        this_ms = (ms_bwd + ms_pre + ms_post) / max(1, n_bwd)
        for mode in (0, 1, 2, 3, 4):
            if mode == det or (d == 256 and mode in (2, 3)):  # partial tiles take d <= 128
                continue
            wsd = fa.bwd_workspace(x["q"], x["k"], causal, mode)
            for _ in range(3):
                fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal, softmax_scale=scale,
                       deterministic=mode, workspace=wsd)
            torch.cuda.synchronize()
            fa.timing_begin()
            for _ in range(args.steps):
                fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal, softmax_scale=scale,
                       deterministic=mode, workspace=wsd)
            kd = fa.timing_end()
            del wsd
            mode_ms = sum(kd[k][1] for k in ("bwd_pre", "bwd_main", "bwd_post")) / args.steps
            extras[f"bwd_mode{mode}_ms"] = mode_ms
            extras[f"bwd_mode{mode}_main_ms"] = kd["bwd_main"][1] / args.steps
            extras[f"bwd_mode{mode}_post_ms"] = kd["bwd_post"][1] / args.steps
            extras[f"bwd_mode{mode}_tflops"] = f_bwd / (mode_ms * 1e-3) / 1e12
            extras[f"bwd_mode{mode}_over_this"] = this_ms / mode_ms
        if d in (64, 128) and args.steps > 0:
            # the forward with fp8 (e4m3) Q and K for the scores, per-tensor descale factors
            qd = float(x["q"].float().abs().max()) / 448.0
            kd = float(x["k"].float().abs().max()) / 448.0
            q8 = (x["q"].float() / qd).to(torch.float8_e4m3fn)
            k8 = (x["k"].float() / kd).to(torch.float8_e4m3fn)
            for _ in range(3):
                fa.fwd_fp8(q8, k8, x["v"], qd, kd, causal=causal, softmax_scale=scale)
            torch.cuda.synchronize()
            fa.timing_begin()
            for _ in range(args.steps):
                fa.fwd_fp8(q8, k8, x["v"], qd, kd, causal=causal, softmax_scale=scale)
            kf = fa.timing_end()["fwd"]
            fp8_ms = kf[1] / max(1, kf[0])
            extras["fp8_fwd_kernel_ms"] = fp8_ms
            extras["fp8_fwd_tflops"] = f_fwd / (fp8_ms * 1e-3) / 1e12
            extras["fp8_fwd_pct_fp8_peak"] = 100.0 * extras["fp8_fwd_tflops"] / MFMA_FP8_PEAK_TFLOPS
            extras["fp8_fwd_speedup_vs_bf16"] = avg_fwd_ms / fp8_ms
            del q8, k8
    if args.variants:
        # forward builds that differ in one compile-time choice: rescale at
        # every growth of a row maximum (tau0), one exponential in four or two
        # from the FMA-unit polynomial (exppoly4, exppoly2)
        from exact_attention_80_amd.build import VARIANTS
        for name in VARIANTS:
            try:
                lib = fa.load_variant(name)
            except ImportError:
                continue
            for _ in range(3):
                fa.fwd(x["q"], x["k"], x["v"], causal=causal, softmax_scale=scale, lib=lib)
            torch.cuda.synchronize()
            fa.timing_begin(lib)
            for _ in range(args.steps):
                fa.fwd(x["q"], x["k"], x["v"], causal=causal, softmax_scale=scale, lib=lib)
            kv = fa.timing_end(lib)["fwd"]
            extras[f"fwd_{name}_kernel_ms"] = kv[1] / max(1, kv[0])
            if "fa_bwd.hip" in VARIANTS[name][0]:
                o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=causal, softmax_scale=scale)
                for tag, lb in (("", None), (f"{name}_", lib)):
                    for _ in range(3):
                        fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal,
                               softmax_scale=scale, deterministic=det, lib=lb)
                    torch.cuda.synchronize()
                    fa.timing_begin(lb)
                    for _ in range(args.steps):
                        fa.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal,
                               softmax_scale=scale, deterministic=det, lib=lb)
                    kb = fa.timing_end(lb)["bwd_main"]
                    extras[f"bwd_main_{tag or 'default_'}kernel_ms"] = kb[1] / max(1, kb[0])

    metric = METRIC
    if (B, N, Hq, Hkv, d, causal) != (2, 8192, 16, 16, 128, True):
        metric = (f"attention fwd+bwd TFLOPs/s (bf16, d={d}, {'causal' if causal else 'non-causal'} "
                  f"N={N}) and % of MFMA peak")
    line = {
        "metric": metric,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{'causal' if causal else 'non-causal'} self-attention forward+backward, "
                        f"B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}, "
                        f"{DQ_MODE_NAMES[det]} "
                        f"dQ reduction",
            "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d, "causal": causal,
            "deterministic": det,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "bwd_kernel (backward main)",
            "achieved": achieved,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
            "traffic": traffic,
        },
        "extras": extras,
    }
    if args.cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(B, N, Hq, Hkv, d, causal, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
