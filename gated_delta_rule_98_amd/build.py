"""Build the HIP library for gfx950: gated_delta_rule_98_amd/libkda.so, and the
benchmark's HBM ceiling probes, gated_delta_rule_98_amd/libkda_ceiling.so.

Sources (csrc/): kda_engine.h holds the device building blocks every kernel
shares; kda_decode.hip, kda_verify.hip, kda_verify_chunk.hip, kda_prefill.hip,
kda_prefill_chunk.hip and kda_state.hip hold the kernels; kda_api.hip holds
the C ABI of include/kda.h. Flags:
  -ffp-contract=off   no implicit FMA contraction: every FMA is written out, so
                      all kernels round identically
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed fp32 instructions (the host pass warns that it
                      does not know the feature; that is expected)
"""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("kda_api.hip", "kda_decode.hip", "kda_verify.hip",
                                           "kda_verify_chunk.hip", "kda_prefill.hip", "kda_prefill_chunk.hip",
                                           "kda_state.hip")]
HEADERS = [os.path.join(CSRC, "kda_engine.h"), os.path.join(ROOT, "include", "kda.h")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
# the benchmark's ceiling probes (csrc/probe/): not part of the KDA library or its C ABI
CEILING_SOURCES = [os.path.join(CSRC, "probe", "kda_ceiling.hip")]
CEILING_LIB = os.path.join(PKG, "libkda_ceiling.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unknown-warning-option",
]


def build(out: str = LIB, extra=(), verbose: bool = False, sources=None) -> str:
    """Compile the library (always recompiles); return its path."""
    tmp = f"{out}.tmp{os.getpid()}"  # per process: concurrent builds never share a file
    cmd = [HIPCC, *FLAGS, *extra, f"-I{INCLUDE}", *(sources or SOURCES), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and (r.stdout or r.stderr):
        print(r.stdout, r.stderr)
    os.replace(tmp, out)
    return out


def build_ceiling(out: str = CEILING_LIB) -> str:
    """Compile the benchmark's ceiling probes (always recompiles); return the path."""
    return build(out=out, sources=CEILING_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ceiling())
