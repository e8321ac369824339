"""Every kernel of the HIP libraries runs from registers alone: the
compiler's per-kernel resource report, which the build writes beside each
library, shows no scratch (register spill) memory for any kernel, and every
kernel fits the 512 VGPRs of a lane."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "zero_sharded_mixed_step_amd")
LIBS = [os.path.join(PKG, "libzero_step.so"), os.path.join(PKG, "libzs_patterns.so")]


def _kernels(path):
    """{mangled kernel name: {field: value}} from the resource remarks."""
    out, cur = {}, None
    with open(path) as fh:
        for ln in fh:
            m = re.search(r"remark: Function Name: (\S+)", ln)
            if m:
                cur = out.setdefault(m.group(1), {})
                continue
            m = re.search(r"remark:\s+(\S[^:]*): (\d+) \[", ln)
            if m and cur is not None:
                cur[m.group(1).strip()] = int(m.group(2))
    return out


@pytest.mark.parametrize("lib", LIBS, ids=os.path.basename)
def test_no_kernel_uses_scratch(lib):
    path = lib + ".resources.txt"
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(lib)} was built without its resource report")
    kernels = _kernels(path)
    assert kernels, "no kernel in the resource report"
    spills = {k: v["ScratchSize [bytes/lane]"] for k, v in kernels.items()
              if v.get("ScratchSize [bytes/lane]", 0) != 0}
    assert not spills, f"kernels using scratch: {spills}"
    assert all(v.get("VGPRs Spill", 0) == 0 for v in kernels.values())
    assert all(0 < v["VGPRs"] <= 512 for v in kernels.values())
