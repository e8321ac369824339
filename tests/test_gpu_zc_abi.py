"""The C ABI driven from C alone: tests/c_abi/abi_roundtrip (built by
__graft_entry__.build()) allocates with the HIP runtime's C API, runs three
gated steps through zero_norm_acc_clear / zero_shard_reduce /
zero_adamw_step (bf16 param, fused MXFP8 pack, skip flag; one call skipped
on an injected inf), compares every output bit for bit with the oracle's
step, and checks the documented status codes of bad arguments.  It runs as
a child process."""
import os
import subprocess

import pytest

from gpu_util import gpu_or_skip

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_roundtrip")


def test_c_program_drives_the_abi():
    gpu_or_skip()
    if not os.path.exists(BIN):
        pytest.skip("tests/c_abi/abi_roundtrip is not built: run __graft_entry__.build()")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"exit {r.returncode}: {r.stderr}"
    assert "abi_roundtrip ok" in r.stdout, r.stdout
