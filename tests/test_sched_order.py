"""Host-side pins of the packed-batch work order ([FA4B] 3.3.2: a
preprocessing step orders the work by per-tile cost; 3.3.1: the cheapest
causal key tiles first for the deterministic reduction).

The scheduler kernel's item, cost and sort-key functions are compiled for the
host (hipcc) and the order they give is checked against definitions written
out here:
  * the items are exactly the tiles of every sequence: forward query tiles of
    `tile` rows (a last tile with at most 32 queries whose keys span nt key
    tiles of 64 is split into chunks of max(32, ceil(nt / 1024)) key tiles
    when that gives two or more), backward key tiles of `tile` keys;
  * a forward tile costs its visible key tiles, a chunk its own key tiles, a
    backward key tile its visible query tiles of 32 rows, with the causal
    diagonal aligned bottom-right (query i sees key j iff j <= i + Lk - Lq);
  * forward and deterministic backward: whole sequences in descending order
    of their largest tile cost (ties by sequence), each sequence's items
    together, the forward from the last query tile (split chunks first, last
    chunk first), the deterministic backward from the last key tile, so every
    key tile comes after all key tiles of its sequence that its ordered dQ
    writes wait for; fast backward: every key tile most expensive first, ties
    by sequence and tile.
The order never changes results (tested on the GPU); these pins guard the
progress argument of the ordered reduction and the load-balancing rule."""

import math
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
FWD_ROWS, BWD_KEYS, KEY_TILE, BQ = 256, 256, 64, 32


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("sched") / "sched_check")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17",
                    os.path.join(HERE, "host", "sched_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def order(exe, mode, causal, lengths):
    tile = FWD_ROWS if mode == 0 else BWD_KEYS
    text = f"{mode} {int(causal)} {tile} {KEY_TILE} {BQ} {len(lengths)}\n"
    text += "\n".join(f"{lq} {lk}" for lq, lk in lengths) + "\n"
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return [tuple(int(v) for v in line.split()) for line in out.splitlines()]


def fwd_items(lq, lk, causal):
    """(idx, cost) of the forward items of one sequence; chunks as -(c + 1)."""
    items = []
    nq = math.ceil(lq / FWD_ROWS)
    for i in range(nq):
        end = max(0, min(lk, (i + 1) * FWD_ROWS + lk - lq)) if causal else lk
        nt = math.ceil(end / KEY_TILE)
        last = i == nq - 1
        if last and lq - i * FWD_ROWS <= 32:
            ct = max(32, math.ceil(nt / 1024))
            n = math.ceil(nt / ct)
            if n >= 2:
                items += [(-(c + 1), min(ct, nt - c * ct)) for c in range(n)]
                continue
        items.append((i, nt))
    return items


def bwd_items(lq, lk, causal):
    nq = math.ceil(lq / BQ)
    out = []
    for j in range(math.ceil(lk / BWD_KEYS)):
        first = max(0, j * BWD_KEYS - (lk - lq)) // BQ
        out.append((j, max(0, nq - first) if causal else nq))
    return out


def check(exe, mode, causal, lengths):
    got = order(exe, mode, causal, lengths)
    per_seq = {s: (fwd_items if mode == 0 else bwd_items)(lq, lk, causal)
               for s, (lq, lk) in enumerate(lengths)}
    want = sorted((s, i, c) for s, items in per_seq.items() for i, c in items)
    assert sorted(got) == want, "items or costs differ from their definition"
    if mode == 1:
        keys = [(-c, s, i) for s, i, c in got]
        assert keys == sorted(keys), "not most expensive first"
        return
    # sequences contiguous, in descending order of their largest tile cost
    seqs = []
    for s, i, c in got:
        if not seqs or seqs[-1] != s:
            assert s not in seqs, f"sequence {s} split"
            seqs.append(s)
    tiles = {s: [i for t, i, c in got if t == s] for s in seqs}
    for s in seqs:
        # last tile first; forward split chunks (-(c + 1)) before the tiles, last chunk first
        want_order = sorted(tiles[s], key=lambda i: (1 << 19) - i - 1 if i < 0 else i,
                            reverse=True)
        assert tiles[s] == want_order, f"sequence {s}: items out of order {tiles[s]}"
    big = [(-max(c for _, c in per_seq[s]), s) for s in seqs]
    assert big == sorted(big), "sequences not in descending order of their largest tile cost"


def random_lengths(rng, n, decode=False):
    out = []
    for _ in range(n):
        lk = int(np.exp(rng.uniform(np.log(1), np.log(20000))))
        lq = int(rng.integers(0, 40)) if decode else (lk if rng.uniform() < 0.5 else int(rng.integers(0, lk + 1)))
        out.append((lq, lk))
    return out


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_order_follows_its_definition(checker, mode, causal):
    rng = np.random.Generator(np.random.PCG64(7 + mode + 3 * causal))
    cases = [
        [(1533, 1533), (12884, 12884), (257, 257), (0, 0), (1, 1)],   # self-attention lengths
        [(1, 700), (1, 33), (3, 1029), (1, 1), (17, 260), (0, 50)],   # decode rows
        [(1, 40000), (3, 9000), (32, 70000)],                          # split one-query tiles
        [(300, 100), (64, 64), (5, 1), (40, 700)],                     # more queries than keys
        [(256, 256)] * 6,                                              # equal costs: ties
    ]
    cases += [random_lengths(rng, int(rng.integers(1, 40)), decode=d) for d in (False, True) for _ in range(6)]
    for lengths in cases:
        check(checker, mode, causal, lengths)
