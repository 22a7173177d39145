"""The compiler's per-kernel resource report, written by the build next to the
library (kernel_resources.json), describes the current sources, and the kernels
of the benchmarked configurations neither spill registers nor use scratch."""
import json
import os

import pytest

from io_aware_exact_08_amd import build

# Kernels the benchmarked configurations run (template arguments: head dim,
# bf16, causal, float32 O, split-KV, bias / head dim, bf16, causal, bias).
HOT = [
    "void fa::fwd_kernel<64, false, false, false, false, false>(fa::FwdArgs)",   # fp16 A100 shape
    "void fa::fwd_kernel<64, false, true, false, false, false>(fa::FwdArgs)",    # fp16 causal
    "void fa::fwd_kernel<128, true, true, true, false, false>(fa::FwdArgs)",     # spiked bf16 causal
    "void fa::fwd_kernel<64, true, true, false, false, false>(fa::FwdArgs)",     # long bf16 causal
    "void fa::bwd_dkdv_kernel<64, false, false, false>(fa::BwdArgs)",
    "void fa::bwd_dkdv_kernel<64, false, true, false>(fa::BwdArgs)",
    "void fa::bwd_dkdv_kernel<64, true, true, false>(fa::BwdArgs)",
    "void fa::bwd_dq_kernel<64, false, false, false>(fa::BwdArgs)",
    "void fa::bwd_dq_kernel<64, false, true, false>(fa::BwdArgs)",
    "void fa::bwd_dq_kernel<64, true, true, false>(fa::BwdArgs)",
]


@pytest.fixture(scope="module")
def report():
    if not os.path.exists(build.RESOURCES):
        pytest.fail("kernel_resources.json is missing: run the build")
    with open(build.RESOURCES) as f:
        return json.load(f)


def test_report_matches_sources(report):
    assert report["sources_sha256_16"] == build.sources_digest(), \
        "kernel_resources.json was written for other sources or flags: rebuild"
    assert report["flags"] == build.HIPCC_FLAGS


@pytest.mark.parametrize("name", HOT)
def test_benchmarked_kernels_do_not_spill(report, name):
    r = report["kernels"].get(name)
    assert r is not None, f"{name} missing from the report"
    assert r["vgpr_spill"] == 0 and r["sgpr_spill"] == 0, (name, r)
    assert r["scratch_bytes_per_lane"] == 0, (name, r)


# The d = 64 / 128 bias forwards count their direct loads by hand; the
# compiler does not see those loads, so it would wait for a spill reload with
# vmcnt(0) and drain the whole pipeline.  All of them must stay spill-free.
BIAS_FWD = [f"void fa::fwd_kernel<{d}, {bf}, {c}, {o}, false, true>(fa::FwdArgs)"
            for d in (64, 128) for bf in ("false", "true") for c in ("false", "true")
            for o in ("false", "true")]


@pytest.mark.parametrize("name", BIAS_FWD)
def test_bias_forwards_do_not_spill(report, name):
    r = report["kernels"].get(name)
    assert r is not None, f"{name} missing from the report"
    assert r["vgpr_spill"] == 0 and r["sgpr_spill"] == 0, (name, r)
    assert r["scratch_bytes_per_lane"] == 0, (name, r)


# The 16-query-wave forward (every unbiased d = 256 one; the non-causal bf16
# d = 128 ones and every bf16 d = 128 split) counts its K/V loads the same way.  Its workgroup
# is eight waves, so it needs two waves per SIMD at d = 256 (one workgroup per
# CU) and four at d = 128 (two).
Q16 = [(256, f"void fa::fwd_q16_kernel<256, {bf}, {c}, {o}, false>(fa::FwdArgs)")
       for bf in ("false", "true") for c in ("false", "true") for o in ("false", "true")]
Q16 += [(256, f"void fa::fwd_q16_kernel<256, {bf}, {c}, false, true>(fa::FwdArgs)")
        for bf in ("false", "true") for c in ("false", "true")]
Q16 += [(128, f"void fa::fwd_q16_kernel<128, true, false, {o}, false>(fa::FwdArgs)")
        for o in ("false", "true")]
Q16 += [(128, f"void fa::fwd_q16_kernel<128, true, {c}, false, true>(fa::FwdArgs)")
        for c in ("false", "true")]


@pytest.mark.parametrize("d,name", Q16)
def test_q16_forwards_do_not_spill(report, d, name):
    r = report["kernels"].get(name)
    assert r is not None, f"{name} missing from the report"
    assert r["vgpr_spill"] == 0 and r["sgpr_spill"] == 0, (name, r)
    assert r["scratch_bytes_per_lane"] == 0, (name, r)
    assert r["occupancy_waves_per_simd"] >= (2 if d == 256 else 4), (name, r)


def test_parser_reads_remarks():
    text = """x.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     AGPRs: 4 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
"""
    assert build.parse_resource_remarks(text) == {
        "_Z1kv": {"vgpr": 128, "agpr": 4, "scratch_bytes_per_lane": 16,
                  "occupancy_waves_per_simd": 2, "vgpr_spill": 3}}
