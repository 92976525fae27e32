"""The C-ABI library loads without a GPU, exports every symbol include/fa.h
declares, and rejects bad arguments on the host before launching anything."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FA_OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
P = 0x10000          # a 16-byte aligned non-null address (never dereferenced)
MIS = 0x10008        # misaligned


@pytest.fixture(scope="module")
def lib():
    from exact_attention_80_amd import build
    if not os.path.exists(build.LIB_PATH):
        build.build()
    L = ctypes.CDLL(build.LIB_PATH)
    p, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [p] * 5 + [i] * 5 + [f, i, p, sz, p]
    L.fa_fwd_fp8.argtypes = [p] * 5 + [i] * 5 + [f, f, f, i, p]
    L.fa_bwd.argtypes = [p] * 9 + [i] * 5 + [f, i, i, p, sz, p]
    L.fa_varlen_fwd.argtypes = [p] * 6 + [i] * 6 + [f, i, p, sz, p]
    L.fa_varlen_bwd.argtypes = [p] * 10 + [i] * 6 + [f, i, i, p, sz, p]
    L.fa_bwd_workspace_size.argtypes = [i] * 7
    L.fa_bwd_workspace_size.restype = sz
    L.fa_fwd_workspace_size.argtypes = [i] * 6
    L.fa_fwd_workspace_size.restype = sz
    L.fa_varlen_fwd_workspace_size.argtypes = [i] * 6
    L.fa_varlen_fwd_workspace_size.restype = sz
    L.fa_varlen_bwd_workspace_size.argtypes = [i] * 7
    L.fa_varlen_bwd_workspace_size.restype = sz
    L.fa_varlen_qk_fwd.argtypes = [p] * 7 + [i] * 8 + [f, i, p, sz, p]
    L.fa_varlen_qk_fwd_fp8.argtypes = [p] * 7 + [i] * 8 + [f, f, f, i, p, sz, p]
    L.fa_varlen_qk_bwd.argtypes = [p] * 11 + [i] * 8 + [f, i, i, p, sz, p]
    L.fa_varlen_qk_fwd_noalloc.argtypes = [p] * 7 + [i] * 8 + [f, i, p]
    L.fa_varlen_qk_fwd_workspace_size.argtypes = [i] * 7
    L.fa_varlen_qk_fwd_workspace_size.restype = sz
    L.fa_varlen_qk_bwd_workspace_size.argtypes = [i] * 8
    L.fa_varlen_qk_bwd_workspace_size.restype = sz
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_last_error.restype = ctypes.c_char_p
    L.fa_workspace_error.argtypes = [p, sz, p, ctypes.POINTER(ctypes.c_uint32)]
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_fp8", "fa_varlen_qk_fwd_fp8", "fa_bwd", "fa_varlen_fwd", "fa_varlen_bwd", "fa_varlen_qk_fwd",
              "fa_varlen_qk_bwd", "fa_fwd_workspace_size",
              "fa_bwd_workspace_size", "fa_status_string", "fa_workspace_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_names(lib):
    assert lib.fa_abi_version() == 1
    assert lib.fa_status_string(0) == b"FA_OK"
    assert lib.fa_status_string(3) == b"FA_ERR_WORKSPACE"
    assert lib.fa_status_string(99) == b"FA_ERR_UNKNOWN"


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, N=128, Hq=2, Hkv=2, d=64, scale=0.125, causal=0):
    return lib.fa_fwd(q, k, v, o, lse, B, N, Hq, Hkv, d, scale, causal, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(lse=None), INVALID),
    (dict(o=MIS), INVALID), (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(N=-3), INVALID),
    (dict(Hq=3, Hkv=2), INVALID), (dict(Hkv=0), INVALID), (dict(causal=2), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(d=96), UNSUPPORTED), (dict(d=512), UNSUPPORTED),
    # per-tile byte ranges are 32-bit: one token's heads must stay below 2^24 elements
    (dict(N=1, Hq=65536, Hkv=1, d=256), UNSUPPORTED),
])
def test_fwd_rejects_bad_arguments(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert lib.fa_last_error()


def fwd_fp8(lib, q8=P, k8=P, v=P, o=P, lse=P, B=1, N=128, Hq=2, Hkv=2, d=64, scale=0.125,
            qd=0.01, kd=0.02, causal=0):
    return lib.fa_fwd_fp8(q8, k8, v, o, lse, B, N, Hq, Hkv, d, scale, qd, kd, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q8=None), INVALID), (dict(k8=None), INVALID), (dict(v=None), INVALID),
    (dict(q8=MIS), INVALID), (dict(B=0), INVALID), (dict(Hq=3, Hkv=2), INVALID),
    (dict(causal=2), INVALID), (dict(scale=0.0), INVALID), (dict(qd=0.0), INVALID),
    (dict(kd=-1.0), INVALID), (dict(qd=float("inf")), INVALID), (dict(kd=float("nan")), INVALID),
    (dict(qd=1e30, kd=1e30), INVALID),
    (dict(d=256), UNSUPPORTED), (dict(d=96), UNSUPPORTED),
])
def test_fwd_fp8_rejects_bad_arguments(lib, kw, status):
    assert fwd_fp8(lib, **kw) == status
    assert lib.fa_last_error()


def bwd(lib, ws=P, ws_bytes=None, det=0, d=64, dq=P, B=1, N=128, Hq=2, Hkv=2):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, N, Hq, Hkv, d, 0, det)
    return lib.fa_bwd(P, P, P, P, P, P, dq, P, P, B, N, Hq, Hkv, d, 0.125, 0, det, ws, ws_bytes, None)


def test_bwd_rejects_bad_arguments(lib):
    assert bwd(lib, ws=None) == WORKSPACE
    assert bwd(lib, ws_bytes=16) == WORKSPACE
    assert bwd(lib, det=5, ws_bytes=1 << 30) == INVALID
    assert bwd(lib, det=-1) == INVALID
    assert bwd(lib, dq=None) == INVALID
    assert bwd(lib, d=80) == UNSUPPORTED
    assert bwd(lib, d=512) == UNSUPPORTED
    # d = 256 takes the atomic, ordered and fixed-point modes only
    assert lib.fa_bwd_workspace_size(1, 128, 2, 2, 256, 1, 0) > 0
    assert lib.fa_bwd_workspace_size(1, 128, 2, 2, 256, 1, 1) > 0
    assert lib.fa_bwd_workspace_size(1, 128, 2, 2, 256, 1, 4) > 0
    assert lib.fa_bwd_workspace_size(1, 128, 2, 2, 256, 1, 2) == 0
    assert lib.fa_bwd_workspace_size(1, 128, 2, 2, 256, 1, 3) == 0
    ws2 = lib.fa_bwd_workspace_size(1, 128, 2, 2, 128, 0, 2)
    assert lib.fa_bwd(P, P, P, P, P, P, P, P, P, 1, 128, 2, 2, 256, 0.1, 0, 2, P, ws2, None) == UNSUPPORTED
    assert bwd(lib, ws=MIS) == INVALID


def test_workspace_sizes(lib):
    B, N, Hq, Hkv, d = 2, 1000, 8, 2, 128
    assert lib.fa_fwd_workspace_size(B, N, Hq, Hkv, d, 1) == 0
    fast = lib.fa_bwd_workspace_size(B, N, Hq, Hkv, d, 1, 0)
    det = lib.fa_bwd_workspace_size(B, N, Hq, Hkv, d, 1, 1)
    assert fast >= B * N * Hq * d * 4 + B * N * Hq * 4  # fp32 dQ accumulator + D
    assert det > fast                                    # plus the semaphores
    # partial-sum mode: one fp32 tile of 32 x d per (query tile, key tile) pair
    # (causal: query tile i meets key tiles 0 .. i / 8), no dQ accumulator
    nq = (N + 31) // 32
    pairs = sum(i // 8 + 1 for i in range(nq))
    part = lib.fa_bwd_workspace_size(B, N, Hq, Hkv, d, 1, 2)
    pairs_bytes = B * Hq * pairs * 32 * d * 4
    assert abs((part - fast) - (pairs_bytes - B * N * Hq * d * 4)) <= 1024
    full = lib.fa_bwd_workspace_size(B, N, Hq, Hkv, d, 0, 2)
    assert full >= B * Hq * nq * ((N + 255) // 256) * 32 * d * 4
    # fused partial-sum mode: the same partial tiles plus one counter per query tile
    fused = lib.fa_bwd_workspace_size(B, N, Hq, Hkv, d, 1, 3)
    assert 0 <= fused - part <= B * Hq * nq * 4 + 512
    # fixed-point mode: the accumulator (int32) plus the K/V maxima (two floats per
    # 256 key rows and key/value head, one per head) and one exponent per row
    fixed = lib.fa_bwd_workspace_size(B, N, Hq, Hkv, d, 1, 4)
    extra = Hkv * ((B * N + 255) // 256) * 8 + Hkv * 4 + B * N * Hq * 4
    assert extra <= fixed - fast <= extra + 3 * 256
    assert lib.fa_bwd_workspace_size(B, N, Hq, Hkv, d, 1, 5) == 0
    assert lib.fa_bwd_workspace_size(B, N, 3, 2, d, 1, 0) == 0
    vf = lib.fa_varlen_fwd_workspace_size(5, 4000, Hq, Hkv, d, 1)
    vb = lib.fa_varlen_bwd_workspace_size(5, 4000, Hq, Hkv, d, 1, 1)
    assert vf >= 256 and vb >= 4000 * Hq * d * 4
    assert lib.fa_varlen_fwd_workspace_size(0, 4000, Hq, Hkv, d, 1) == 0


def test_varlen_rejects_bad_arguments(lib):
    ws_n = lib.fa_varlen_fwd_workspace_size(3, 300, 2, 2, 64, 1)
    assert lib.fa_varlen_fwd(P, P, P, P, P, P, 0, 300, 0, 2, 2, 64, 0.1, 1, P, ws_n, None) == INVALID
    assert lib.fa_varlen_fwd(P, P, P, P, P, None, 3, 300, 0, 2, 2, 64, 0.1, 1, P, ws_n, None) == INVALID
    assert lib.fa_varlen_fwd(P, P, P, P, P, P, 3, 300, 0, 2, 2, 64, 0.1, 1, P, 8, None) == WORKSPACE
    assert lib.fa_varlen_fwd(P, P, P, P, P, P, 3, 300, -1, 2, 2, 64, 0.1, 1, P, ws_n, None) == INVALID
    wb = lib.fa_varlen_bwd_workspace_size(3, 300, 2, 2, 64, 1, 1)
    assert lib.fa_varlen_bwd(P, P, P, P, P, P, P, P, P, P, 3, 300, 0, 2, 2, 64, 0.1, 1, 1, P, wb - 1,
                             None) == WORKSPACE
    assert lib.fa_varlen_bwd(P, P, P, P, P, P, P, P, P, P, 3, 0, 0, 2, 2, 64, 0.1, 1, 1, P, wb,
                             None) == INVALID
    # the partial-sum dQ reduction is dense-only; the fixed-point one is not
    assert lib.fa_varlen_bwd_workspace_size(3, 300, 2, 2, 64, 1, 2) == 0
    assert lib.fa_varlen_bwd_workspace_size(3, 300, 2, 2, 64, 1, 4) > wb
    assert lib.fa_varlen_bwd(P, P, P, P, P, P, P, P, P, P, 3, 300, 0, 2, 2, 64, 0.1, 1, 2, P, wb,
                             None) == UNSUPPORTED
    assert lib.fa_varlen_bwd(P, P, P, P, P, P, P, P, P, P, 3, 300, 0, 2, 2, 64, 0.1, 1, 3, P, wb,
                             None) == UNSUPPORTED


def test_varlen_qk_sizes_and_bad_arguments(lib):
    # equal lengths: the same workspace as the single-offset calls
    assert (lib.fa_varlen_qk_fwd_workspace_size(3, 300, 300, 2, 2, 64, 1)
            == lib.fa_varlen_fwd_workspace_size(3, 300, 2, 2, 64, 1))
    for det in (0, 1, 4):
        assert (lib.fa_varlen_qk_bwd_workspace_size(3, 300, 300, 4, 2, 64, 1, det)
                == lib.fa_varlen_bwd_workspace_size(3, 300, 4, 2, 64, 1, det))
    # the backward workspace grows with the query side (dQ accumulator, D, LSE)
    # and, when a group is split, with the key side (dK/dV partials)
    small = lib.fa_varlen_qk_bwd_workspace_size(3, 30, 3000, 2, 2, 128, 1, 0)
    big = lib.fa_varlen_qk_bwd_workspace_size(3, 3000, 3000, 2, 2, 128, 1, 0)
    assert small >= 30 * 2 * 128 * 4 and big - small >= (3000 - 30) * 2 * 128 * 4
    assert lib.fa_varlen_qk_bwd_workspace_size(3, 300, 0, 2, 2, 64, 1, 0) == 0
    assert lib.fa_varlen_qk_bwd_workspace_size(3, 300, 400, 2, 2, 64, 1, 2) == 0
    wf = lib.fa_varlen_qk_fwd_workspace_size(3, 30, 400, 2, 2, 64, 1)
    args = [P] * 7 + [3, 30, 400, 0, 0, 2, 2, 64, 0.1, 1, P, wf, None]
    a = list(args); a[6] = None                    # cu_seqlens_k
    assert lib.fa_varlen_qk_fwd(*a) == INVALID
    a = list(args); a[5] = None                    # cu_seqlens_q
    assert lib.fa_varlen_qk_fwd(*a) == INVALID
    a = list(args); a[9] = 0                       # total_k
    assert lib.fa_varlen_qk_fwd(*a) == INVALID
    a = list(args); a[11] = -1                     # max_seqlen_k
    assert lib.fa_varlen_qk_fwd(*a) == INVALID
    a = list(args); a[18] = 8                      # workspace too small
    assert lib.fa_varlen_qk_fwd(*a) == WORKSPACE
    wb = lib.fa_varlen_qk_bwd_workspace_size(3, 30, 400, 2, 2, 64, 1, 1)
    bargs = [P] * 11 + [3, 30, 400, 0, 0, 2, 2, 64, 0.1, 1, 1, P, wb, None]
    b = list(bargs); b[10] = None                  # cu_seqlens_k
    assert lib.fa_varlen_qk_bwd(*b) == INVALID
    b = list(bargs); b[21] = 2                     # partial-sum mode is dense-only
    assert lib.fa_varlen_qk_bwd(*b) == UNSUPPORTED
    b = list(bargs); b[23] = wb - 1
    assert lib.fa_varlen_qk_bwd(*b) == WORKSPACE


def test_workspace_error_rejects_null(lib):
    assert lib.fa_workspace_error(None, 0, None, None) == INVALID


def test_binding_has_no_fallback():
    """The Python binding only marshals arguments; it loads the HIP library and
    never imports the oracle."""
    src = open(os.path.join(ROOT, "exact_attention_80_amd", "fa.py")).read()
    assert "oracle" not in src
    assert "numpy" not in src


def test_varlen_qk_fwd_fp8_rejects_bad_arguments(lib):
    ws_n = lib.fa_varlen_qk_fwd_workspace_size(2, 100, 3000, 4, 2, 128, 1)
    assert ws_n > 0

    def call(q8=P, cuq=P, ws=P, nbytes=ws_n, d=128, qd=0.01, kd=0.02, nseq=2):
        return lib.fa_varlen_qk_fwd_fp8(q8, P, P, P, P, cuq, P, nseq, 100, 3000, 0, 0, 4, 2, d,
                                        0.125, qd, kd, 1, ws, nbytes, None)
    assert call(q8=None) == INVALID
    assert call(cuq=None) == INVALID
    assert call(nseq=0) == INVALID
    assert call(qd=0.0) == INVALID
    assert call(kd=float("inf")) == INVALID
    assert call(d=256) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE
    assert call(nbytes=16) == WORKSPACE

def test_noalloc_entry_point_checks_on_the_host(lib):
    """fa_varlen_qk_fwd_noalloc rejects bad arguments and problems whose
    workspace exceeds its static scratch (64 MiB) before touching the device."""
    limit = 64 << 20
    text = open(HEADER).read()
    assert "#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)" in text

    def call(nseq=3, tq=30, tk=400, hq=2, hkv=2, d=64, cuq=P, q=P, maxk=0):
        return lib.fa_varlen_qk_fwd_noalloc(q, P, P, P, P, cuq, P, nseq, tq, tk, 0, maxk, hq, hkv,
                                            d, 0.1, 1, None)
    assert call(nseq=0) == INVALID
    assert call(maxk=-1) == INVALID
    assert call(cuq=None) == INVALID
    assert call(q=None) == INVALID
    assert call(tk=0) == INVALID
    assert call(d=96) == UNSUPPORTED
    # 400 sequences of 2048 keys, 64 heads of d = 256: the split-tile partials
    # alone need far more than the scratch
    assert lib.fa_varlen_qk_fwd_workspace_size(400, 400, 400 * 2048, 64, 8, 256, 1) > limit
    assert call(nseq=400, tq=400, tk=400 * 2048, hq=64, hkv=8, d=256) == WORKSPACE
    assert b"no-allocation limit" in lib.fa_last_error()
