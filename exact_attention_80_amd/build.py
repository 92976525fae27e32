"""Compile the HIP sources into the in-tree shared library libfa_mi355x.so (gfx950 only).

Every call recompiles all sources (in parallel) and relinks.  Objects go to
exact_attention_80_amd/_build/, the library next to this file.

Besides the library itself one variant is built for the tests:
libfa_mi355x_tau0.so, whose forward rescales its accumulator on every growth
of a row maximum (rescale threshold 0 instead of 8 log2 units).  Its results
must agree with the default build's within rounding; the product never loads
it.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_sched.hip"]

# name -> (sources rebuilt for the variant, extra flags for them)
VARIANTS = {
    "tau0": (["fa_fwd.hip"], ["-DFA_RESCALE_TAU=0.0f"]),
    # one exponential in four (or two) from the FMA-unit polynomial
    "exppoly4": (["fa_fwd.hip"], ["-DFA_EXP_POLY_EVERY=4"]),
    "exppoly2": (["fa_fwd.hip"], ["-DFA_EXP_POLY_EVERY=2"]),
    # the d = 64 backward with 64 keys per wave (4 waves, one per SIMD)
    "bwd64keys": (["fa_bwd.hip"], ["-DFA_BWD_KEY_BLOCKS=2"]),
}

# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def variant_path(name: str) -> str:
    return os.path.join(HERE, f"libfa_mi355x_{name}.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def _link(cc, objs, path, verbose):
    tmp = path + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, path)


def build(verbose: bool = False, jobs: int | None = None, extra_flags: list[str] | None = None,
          variants: bool = True) -> str:
    """Compile all sources for gfx950 and link the library (and, unless
    variants is False, the test variants); returns the library's path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = HIP_FLAGS + list(extra_flags or [])
    objs = {}
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs[src] = obj
        cmds.append([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    var_objs = {}
    if variants:
        for name, (srcs, vflags) in VARIANTS.items():
            var_objs[name] = dict(objs)
            for src in srcs:
                obj = os.path.join(BUILD_DIR, src.replace(".hip", f"_{name}.o"))
                var_objs[name][src] = obj
                cmds.append([cc, *flags, *vflags, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = jobs or min(len(cmds), max(1, (os.cpu_count() or 2) // 2))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    _link(cc, [objs[s] for s in SOURCES], LIB_PATH, verbose)
    for name, vo in var_objs.items():
        _link(cc, [vo[s] for s in SOURCES], variant_path(name), verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
