"""The build's resource check (CPU only): hipcc's kernel-resource-usage remarks are parsed per kernel, and the
built library's kernels use no scratch memory."""
import os

import pytest

from sparse_kv_cache_sfi_amd import build as B

SAMPLE = """\
x.hip:50:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]
   50 | __global__ void k() {
      | ^
x.hip:50:1: remark:     VGPRs: 10 [-Rpass-analysis=kernel-resource-usage]
x.hip:50:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
In file included from y.hip:2:
x.h:60:1: remark: Function Name: _Z1jv [-Rpass-analysis=kernel-resource-usage]
   60 | __global__ void j() {
      | ^
x.h:60:1: remark:     ScratchSize [bytes/lane]: 48 [-Rpass-analysis=kernel-resource-usage]
In file included from y.hip:2:
x.h:10:5: warning: unused variable 'u' [-Wunused-variable]
"""


def test_resource_remarks_are_parsed_per_kernel():
    other, usage = B._resource_usage(SAMPLE)
    assert usage == {"_Z1kv": {"VGPRs": "10", "ScratchSize [bytes/lane]": "0"},
                     "_Z1jv": {"ScratchSize [bytes/lane]": "48"}}
    # a real diagnostic keeps its include context; the remarks and their source lines are gone
    assert other.splitlines() == ["In file included from y.hip:2:",
                                  "x.h:10:5: warning: unused variable 'u' [-Wunused-variable]"]


def test_built_kernels_use_no_scratch():
    path = os.path.join(B.BUILD, "resource_usage.txt")
    if not os.path.exists(path):
        pytest.skip("library not built here")
    lines = [l for l in open(path) if l.strip()]
    assert lines, "no kernels recorded"
    for line in lines:
        assert "ScratchSize [bytes/lane]=0" in line and "VGPRs Spill=0" in line, line.split()[0]
