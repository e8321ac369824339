"""Build libzero_step.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Floating-point flags are part of the contract: no contraction of a*b+c into
fma unless written, IEEE-correct binary32 division and square root, denormals
kept, and no packed-fp32 instructions.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzero_step.so")
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("zs_kernels.hip", "zs_unfused.hip", "zs_abi.hip", "zs_noalloc.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


# The bare access patterns the benchmark measures as ceilings (not part of
# the step's ABI; bench.py alone loads it).
PATTERNS_LIB = os.path.join(HERE, "libzs_patterns.so")
PATTERNS_SOURCES = [os.path.join(HERE, "csrc", "zs_patterns.hip")]


def _compile(sources, out, defines, verbose):
    """Compiles `sources` into `out`, and writes the compiler's per-kernel
    resource report (registers, scratch, occupancy) to out + RESOURCES."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines],
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           "-Rpass-analysis=kernel-resource-usage", "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    remarks = [ln for ln in r.stderr.splitlines() if "kernel-resource-usage" in ln]
    rest = "\n".join(ln for ln in r.stderr.splitlines() if "kernel-resource-usage" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{rest}")
    if verbose and rest.strip():
        print(rest, flush=True)
    with open(out + RESOURCES, "w") as fh:
        fh.write("\n".join(remarks) + "\n")
    os.replace(tmp, out)
    return out


# Suffix of the per-kernel resource report written beside each library.
RESOURCES = ".resources.txt"


def build(verbose: bool = False, out: str = LIB, defines=(), patterns: bool = True) -> str:
    """libzero_step.so (and, unless patterns=False, libzs_patterns.so)."""
    _compile(SOURCES, out, defines, verbose)
    if patterns:
        _compile(PATTERNS_SOURCES, PATTERNS_LIB, (), verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
