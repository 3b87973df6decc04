"""Build libffd.so (gfx950) and the measurement aid libffd_probe.so in-tree with hipcc.

    python -m long_context_decoding_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libffd.so"
# ffd_kernels_stream.hip compiles the second half of ffd_kernels.hip (the streaming-policy decode
# kernels); the translation units compile in parallel
SOURCES = [CSRC / "ffd_kernels.hip", CSRC / "ffd_kernels_stream.hip", CSRC / "ffd_scratch.hip",
           CSRC / "ffd_api.cpp"]
HEADERS = [CSRC / "ffd_internal.h", ROOT / "include" / "ffd.h"]
PROBE_LIB = PKG / "libffd_probe.so"
PROBE_SOURCES = [CSRC / "probe.hip"]
ARCH = os.environ.get("FFD_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed fp32 math in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the selection arithmetic must not be contracted into FMAs (explicit __f*_rn ops are used
    # there as well); attention math uses explicit fmaf where a fused op is wanted
    "-ffp-contract=off",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (Path(c).exists() or c == "hipcc"):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def _compile(lib: Path, sources, verbose: bool) -> Path:
    """Each source to an object (in parallel), then one shared library."""
    tmp = lib.with_suffix(".so.tmp")
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="ffd_build_") as td:
        objs = [str(Path(td) / (Path(src).name + ".o")) for src in sources]
        with ThreadPoolExecutor(max_workers=len(sources)) as ex:
            list(ex.map(lambda so: _run([hipcc(), *compile_flags, "-c", "-o", so[1], str(so[0])],
                                        verbose), zip(sources, objs)))
        _run([hipcc(), *HIPCC_FLAGS, "-o", str(tmp), *objs], verbose)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> Path:
    """Compile libffd.so and libffd_probe.so; returns the path of libffd.so."""
    _compile(LIB, SOURCES, verbose)
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
