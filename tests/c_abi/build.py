"""Compile the C-ABI round-trip test program tests/c_abi/abi_roundtrip (test
infrastructure: it links libzero_step.so, the CPU oracle and the host input
generator; run by tests/test_gpu_zc_abi.py).  Plain C11 with gcc against the
HIP runtime's C API; the libraries are found next to the tree through
$ORIGIN-relative run paths."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "abi_roundtrip")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "zero_sharded_mixed_step_amd")
    orc = os.path.join(ROOT, "oracle")
    syn = os.path.join(ROOT, "synth")
    rpath = ":".join(["$ORIGIN/../../zero_sharded_mixed_step_amd", "$ORIGIN/../../oracle",
                      "$ORIGIN/../../synth", f"{ROCM}/lib"])
    tmp = OUT + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", orc, "-I", syn, "-I", f"{ROCM}/include",
           os.path.join(HERE, "abi_roundtrip.c"), "-o", tmp,
           "-L", pkg, "-lzero_step", "-L", orc, "-loracle", "-L", syn, "-lsynth_cpu",
           "-L", f"{ROCM}/lib", "-lamdhip64", "-lm", f"-Wl,-rpath,{rpath}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
