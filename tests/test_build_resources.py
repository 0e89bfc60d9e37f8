"""Register use of the library's kernels, as hipcc reported it at the last
build (bit_weight_gemm_amd/build.py writes _build/resource_usage.json): no
kernel of the product, the quantisers or the packer may use scratch memory
(spilled registers or private arrays), and none may exceed the 512 VGPRs of
a gfx950 lane."""
import json
import os

import pytest

from bit_weight_gemm_amd import build as hipbuild


def _usage():
    if not os.path.exists(hipbuild.RESOURCES):
        pytest.skip("the library has not been built here (run __graft_entry__.build())")
    with open(hipbuild.RESOURCES) as f:
        return json.load(f)


def test_every_source_reported():
    usage = _usage()
    for src in hipbuild.SOURCES:
        if src.endswith(".hip"):
            assert src in usage, f"{src}: no resource report"
    assert any("fused_gemv_kernel" in k for k in usage["k_fused_gemv.hip"])
    assert any("mfma_product_kernel" in k for k in usage["k_fused_mfma.hip"])


# The refit's panel kernel (one workgroup, 32 launches per decomposition, off
# the product's path) keeps each thread's row of the forward substitution,
# 32 doubles, partly in scratch.
SCRATCH_ALLOWED = {"_ZN6biloco22peel_chol_panel_kernelEPdiidPi"}


def test_no_kernel_uses_scratch():
    bad = {k: v for src in _usage().values() for k, v in src.items()
           if v.get("scratch_bytes_per_lane", 0) > 0 and k not in SCRATCH_ALLOWED}
    assert not bad, f"kernels with scratch memory: {sorted(bad)}"


def test_vgprs_within_a_lane():
    for src in _usage().values():
        for k, v in src.items():
            assert 0 < v.get("vgprs", 1) <= 512, k
