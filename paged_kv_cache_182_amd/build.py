"""Builds libpkv.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc,
and libpkv_probe.so, the benchmark's read-bandwidth probes (not part of the
decode library or its ABI).

    python -m paged_kv_cache_182_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = ["pkv_kernels.hip", "pkv_write.hip", "pkv_prefill.hip", "pkv_select.hip", "pkv_api.cpp"]
PROBE_LIB = os.path.join(HERE, "libpkv_probe.so")
PROBE_SOURCES = ["read_probe.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no AGPR copies around the online-softmax rescale
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpkv.so")


def build(verbose: bool = False, out: str = LIB, extra: tuple = (), sources=None) -> str:
    """Compile the decode library's sources into libpkv.so (always recompiles).
    Returns its path. `extra` adds compiler flags (for example -D variants of
    a tuning macro); `sources` replaces the source list."""
    tmp = out + ".tmp"
    srcs = SOURCES if sources is None else sources
    cmd = [hipcc(), *FLAGS, *extra, *[os.path.join(CSRC, s) for s in srcs], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    noise = [ln for ln in (res.stdout + res.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    """Compile libpkv_probe.so (the benchmark's read probes)."""
    return build(verbose, out=PROBE_LIB, sources=PROBE_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
