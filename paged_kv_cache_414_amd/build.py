"""Build ``libpa.so`` (the C-ABI library with the gfx950 HIP kernels) in-tree, and
``libpa_debug.so``: the same kernels with the host sources compiled with
PA_DEBUG_CHECKS=1 (every entry point checks the device data it hands to a kernel).

    python -m paged_kv_cache_414_amd.build          # build both
    python -m paged_kv_cache_414_amd.build --asm    # also dump gfx950 assembly to _build/

Each source is compiled to an object of its own under _build/obj (in parallel); the
HIP sources' objects serve both libraries.
"""

from __future__ import annotations

import argparse
import concurrent.futures
import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libpa.so"
DEBUG_LIB = PKG / "libpa_debug.so"
BUILD_DIR = ROOT / "_build"
OBJ_DIR = BUILD_DIR / "obj"

# sources whose code does not depend on PA_DEBUG_CHECKS, then those that do
KERNEL_SOURCES = [CSRC / "pa_kernels.hip", CSRC / "pa_copy.hip", CSRC / "pa_stage.hip", CSRC / "pa_noalloc.hip",
                  CSRC / "pa_blocks.cpp"]
CHECKED_SOURCES = [CSRC / "pa_api.cpp", CSRC / "pa_step.cpp", CSRC / "pa_debug.cpp"]
SOURCES = KERNEL_SOURCES + CHECKED_SOURCES
HEADERS = [INCLUDE / "pa.h", INCLUDE / "pa_blocks.h", INCLUDE / "pa_step.h", CSRC / "pa_launch.h", CSRC / "pa_status.h",
           CSRC / "pa_debug.h"]

OFFLOAD_ARCH = "gfx950"

# Packed fp32 instructions are switched off for all device code.
COMMON_FLAGS = [
    f"--offload-arch={OFFLOAD_ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError(f"hipcc not found (looked for {path})")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(str(c) for c in cmd), flush=True)
    res = subprocess.run([str(c) for c in cmd], capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build failed: {' '.join(str(c) for c in cmd[:2])} ...")
    # keep warnings visible, but hide the host pass's note about the device-only feature
    noise = "is not a recognized feature for this target"
    text = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if text.strip() and verbose:
        sys.stderr.write(text + "\n")


def _compile(src: pathlib.Path, obj: pathlib.Path, defines, verbose):
    _run([hipcc(), *COMMON_FLAGS, *defines, "-c", "-o", obj, src], verbose)
    return obj


def _link(objs, lib: pathlib.Path, verbose):
    tmp = lib.with_suffix(".so.tmp")
    _run([hipcc(), *COMMON_FLAGS, "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, jobs: int | None = None) -> pathlib.Path:
    """Compile every source and link ``libpa.so`` and ``libpa_debug.so`` next to this
    file (always rebuilds); returns the path of ``libpa.so``."""
    OBJ_DIR.mkdir(parents=True, exist_ok=True)
    tasks = [(src, OBJ_DIR / f"{src.name}.o", []) for src in SOURCES]
    tasks += [(src, OBJ_DIR / f"{src.name}.debug.o", ["-DPA_DEBUG_CHECKS=1"]) for src in CHECKED_SOURCES]
    jobs = jobs or min(len(tasks), os.cpu_count() or 1, 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        futures = [pool.submit(_compile, src, obj, defs, verbose) for src, obj, defs in tasks]
        objs = [f.result() for f in futures]
    kernel_objs = objs[:len(KERNEL_SOURCES)]
    release = objs[:len(SOURCES)]
    debug = kernel_objs + objs[len(SOURCES):]
    _link(release, LIB, verbose)
    _link(debug, DEBUG_LIB, verbose)
    return LIB


def dump_asm(verbose: bool = False) -> pathlib.Path:
    """Write the gfx950 assembly of the kernels to _build/pa_kernels-gfx950.s."""
    BUILD_DIR.mkdir(exist_ok=True)
    out = BUILD_DIR / f"pa_kernels-{OFFLOAD_ARCH}.s"
    cmd = [hipcc(), *COMMON_FLAGS, "--cuda-device-only", "-S", "-o", out, CSRC / "pa_kernels.hip"]
    _run(cmd, verbose)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose))
    if args.asm:
        print(dump_asm(verbose=args.verbose))


if __name__ == "__main__":
    main()
