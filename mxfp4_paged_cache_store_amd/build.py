"""Build libmxstore.so (the HIP kernels + C ABI) for gfx950 with hipcc.

The library is built in-tree, under ``mxfp4_paged_cache_store_amd/_build/``,
so it travels with the source tree.  ``python -m
mxfp4_paged_cache_store_amd.build`` (or ``build()``) always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libmxstore.so")
INCLUDE_DIR = os.path.join(ROOT_DIR, "include")

# The benchmark's memory-system probes (bench_probes.hip beside bench.py),
# built into a library of their own: not part of libmxstore.
PROBE_SRC = os.path.join(ROOT_DIR, "bench_probes.hip")
PROBE_LIB_PATH = os.path.join(BUILD_DIR, "libmxprobe.so")

SOURCES = ["mxstore_abi.hip", "mxfp4_store.hip", "mxfp4_dequant.hip", "rope_insert.hip",
           "ring_rows.hip", "compress_norm.hip", "sparse_attn.hip"]

# -ffp-contract=off: every multiply and add rounds once (the RoPE arithmetic
#   and the x*2^-e + 0.0 sign fix-up depend on it).
# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 (kept out on these parts).
# fp32 denormals stay enabled (HIP's default; nothing here asks for FTZ).
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libmxstore")
    return path


def build(verbose: bool = False, extra_flags: list[str] | None = None,
          out: str | None = None) -> str:
    """Compile libmxstore.so from the csrc/ sources (always recompiles)."""
    return _compile([os.path.join(CSRC, s) for s in SOURCES], out or LIB_PATH, verbose,
                    extra_flags)


def build_probes(verbose: bool = False) -> str:
    """Compile the benchmark's probe library, libmxprobe.so."""
    return _compile([PROBE_SRC], PROBE_LIB_PATH, verbose, None)


def _compile(srcs: list[str], out: str, verbose: bool, extra_flags: list[str] | None) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE_DIR, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 target feature; that warning
    # is expected and not shown.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and "ignoring feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probes(verbose="-v" in sys.argv))
