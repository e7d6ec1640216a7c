"""Build libsfa.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

    python -m mla_sparse_top_amd.build          # or: from mla_sparse_top_amd.build import build

Always compiles (no up-to-date check). The library lands next to this file so that it travels
with the source tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libsfa.so")
# measurement context only (an MFMA throughput probe), kept out of the attention library
PROBE_LIB_PATH = os.path.join(PKG, "libsfa_probe.so")
PROBE_SOURCES = ["probe_mfma.hip"]
SOURCES = ["sfa_kernels.hip", "sfa_host.cpp", "sfa_noalloc.hip", "indexer_kernels.hip", "indexer_host.cpp",
           "cache_kernels.hip", "cache_host.cpp", "compress_kernels.hip", "compress_host.cpp", "prolog_kernels.hip",
           "prolog_host.cpp"]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def build_command(out_path: str, sources=None) -> list:
    sources = SOURCES if sources is None else sources
    return [
        hipcc_path(),
        "--offload-arch=gfx950",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # keep packed-fp32 VALU instructions out of the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE,
        "-I", CSRC,
        *[os.path.join(CSRC, s) for s in sources],
        "-o", out_path,
    ]


def _build_one(lib_path: str, sources, verbose: bool) -> str:
    tmp = lib_path + ".tmp"
    cmd = build_command(tmp, sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False) -> str:
    """Builds libsfa.so (the attention, indexer and cache-write kernels behind the C ABI) and
    libsfa_probe.so (the MFMA throughput probe used for measurement context)."""
    _build_one(PROBE_LIB_PATH, PROBE_SOURCES, verbose)
    return _build_one(LIB_PATH, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
