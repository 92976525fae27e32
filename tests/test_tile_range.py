"""Host-side check of the byte range that bounds every direct tile copy.

The kernels copy a tile of at most `tile_rows` rows through a buffer
descriptor whose 32-bit range ends after the tile's last valid row; rows past
the sequence end read as zeros.  The range must cover every valid row of the
tile and must not wrap, also when the whole remaining sequence would span more
than 4 GiB (a long sequence with many heads).  The device function itself is
compiled for the host here (hipcc) and checked against the definition:
(min(len - row0, tile_rows) - 1) * row_bytes + data_bytes, or 0 for an empty
tile."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("tile_range") / "tile_range_check")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17",
                    os.path.join(HERE, "host", "tile_range_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def ranges(exe, cases):
    text = "".join(" ".join(map(str, c)) + "\n" for c in cases)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return [int(x) for x in out.split()]


def expected(row0, n, row_bytes, data_bytes, tile_rows):
    if row0 >= n:
        return 0
    return (min(n - row0, tile_rows) - 1) * row_bytes + data_bytes


def test_range_matches_definition_and_never_wraps(checker):
    N = (1 << 20) + 32
    cases = [
        # K/V tile of 64 keys at key 2^19 of a 2^20+32-token sequence, 32 heads
        # of d = 128 bf16 (a 8 KiB row): the rest of the sequence spans 4.3 GB
        (1 << 19, N, 32 * 128 * 2, 128 * 2, 64),
        # the last, ragged tile of that sequence (32 rows)
        (N - 32, N, 32 * 128 * 2, 128 * 2, 64),
        # backward Q/dO tile of 32 rows, 64 query heads of d = 256
        (12345 * 32, 1 << 20, 64 * 256 * 2, 256 * 2, 32),
        # fp8 K rows (one byte per element)
        (640, 700, 8 * 128, 128, 64),
        # empty tile, single-row sequence, exactly full tile
        (64, 64, 4096, 256, 64),
        (0, 1, 4096, 256, 64),
        (0, 64, 4096, 256, 64),
    ]
    got = ranges(checker, cases)
    for c, g in zip(cases, got):
        e = expected(*c)
        assert e < 2 ** 32, c
        assert g == e, (c, g, e)
    # the first example covers all 64 rows of its tile
    assert got[0] == 63 * 32 * 128 * 2 + 128 * 2
