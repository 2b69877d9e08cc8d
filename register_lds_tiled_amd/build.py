"""Build libsgemm_mi355x.so in place from csrc/*.hip with hipcc for gfx950.

Usage: ``python -m register_lds_tiled_amd.build`` (or call ``build()``).
Objects go to ``register_lds_tiled_amd/_build/``; the library is written next
to this file, where ``binding`` loads it from.

The same sources also build the debug variant libsgemm_mi355x_ldspoison.so
(-DSGEMM_LDS_POISON: every kernel poisons each LDS location with NaN between
the barrier that retires it and its refill; csrc/lds_poison.h).  Its objects
go to ``_build/ldspoison/``.  ``build()`` makes both, compiling in parallel.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsgemm_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
# Packed fp32 (v_pk_*_f32) code generation is switched off for every device
# pass; the host pass warns that it does not know the feature, harmlessly.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# variant -> (library, extra flags, object directory)
VARIANTS = {
    "release": (LIB, [], OBJ),
    "ldspoison": (os.path.join(HERE, "libsgemm_mi355x_ldspoison.so"), ["-DSGEMM_LDS_POISON"],
                  os.path.join(OBJ, "ldspoison")),
}


def _compile(src: str, extra=(), objdir: str = OBJ) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # Known, checked diagnostics: the host pass does not know the packed-fp32
    # feature; the DMA asm names M0, which tests/test_isa.py shows nothing
    # else in the kernels uses.  Anything else is printed.
    known = ("packed-fp32-ops", "reserved registers: m0",
             "Reserved registers on the clobber list")
    other = [l for l in r.stderr.splitlines()
             if ("warning:" in l or "error:" in l or "note:" in l)
             and not any(k in l for k in known)]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    if other:
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = True, variants=("release", "ldspoison")) -> str:
    """Compile every csrc/*.hip and link the shared library of each variant
    (always rebuilds).  Returns the release library's path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = []
    for v in variants:
        lib, extra, objdir = VARIANTS[v]
        os.makedirs(objdir, exist_ok=True)
        jobs += [(v, src, extra, objdir) for src in srcs]
    # the largest translation units first, so they do not finish last
    jobs.sort(key=lambda j: -os.path.getsize(j[1]))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        futs = [(j[0], ex.submit(_compile, j[1], j[2], j[3])) for j in jobs]
        objs = {v: [] for v in variants}
        for v, f in futs:
            objs[v].append(f.result())
    for v in variants:
        lib = VARIANTS[v][0]
        tmp = lib + ".tmp"
        subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *sorted(objs[v]), "-o", tmp],
                       check=True)
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
