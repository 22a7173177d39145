"""Host logic of bench.py (no GPU): the copy-calibrated HBM traffic summary
and the rule that a stored summary only counts for the kernel sources it was
taken on."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy(tmp_path):
    # a 4 MiB copy that FETCH_SIZE reads as half its bytes and WRITE_SIZE as all
    fetch = [("__amd_rocclr_copyBuffer", 2048.0),
             ("void fa::fwd_kernel<64, false, false, false, false, false>(fa::FwdArgs)", 100.0),
             ("void fa::fwd_kernel<64, false, false, false, false, false>(fa::FwdArgs)", 300.0),
             ("void fa::bwd_dq_kernel<64, false, false, false>(fa::BwdArgs)", 50.0)]
    write = [("__amd_rocclr_copyBuffer", 4096.0),
             ("void fa::fwd_kernel<64, false, false, false, false, false>(fa::FwdArgs)", 10.0),
             ("void fa::fwd_kernel<64, false, false, false, false, false>(fa::FwdArgs)", 30.0),
             ("void fa::bwd_dq_kernel<64, false, false, false>(fa::BwdArgs)", 5.0)]
    fp, wp, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _write(fp, "FETCH_SIZE", fetch)
    _write(wp, "WRITE_SIZE", write)
    bench.traffic_summary(str(fp), str(wp), str(out), 4)
    rec = json.load(open(out))
    assert rec["FETCH_SIZE_factor"] == 2.0 and rec["WRITE_SIZE_factor"] == 1.0
    assert rec["counter_kib_per_launch"]["fwd_kernel"] == {"FETCH_SIZE": 200.0, "WRITE_SIZE": 20.0}
    # average per launch, KiB -> bytes, each counter scaled by its own factor
    assert rec["hbm_bytes_per_launch"]["fwd_kernel"] == (200 * 2 + 20) * 1024
    assert rec["hbm_bytes_per_launch"]["bwd_dq_kernel"] == (50 * 2 + 5) * 1024
    assert "bwd_dkdv_kernel" not in rec["hbm_bytes_per_launch"]
    assert rec["sources_sha256_16"] == bench.sources_digest()


def test_traffic_counts_only_for_the_same_sources(tmp_path, monkeypatch):
    path = tmp_path / "t.json"
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(path))
    assert bench.traffic_from_profile("fwd_kernel") is None  # missing file
    rec = {"sources_sha256_16": bench.sources_digest(), "hbm_bytes_per_launch": {"fwd_kernel": 123}}
    path.write_text(json.dumps(rec))
    assert bench.traffic_from_profile("fwd_kernel") == 123
    assert bench.traffic_from_profile("bwd_dq_kernel") is None
    rec["sources_sha256_16"] = "0" * 16  # taken on other kernel sources
    path.write_text(json.dumps(rec))
    assert bench.traffic_from_profile("fwd_kernel") is None


def test_digest_covers_every_file_with_device_code():
    csrc = os.path.join(ROOT, "io_aware_exact_08_amd", "csrc")
    device = set()
    for f in os.listdir(csrc):
        if f.endswith((".hip", ".hpp")):
            text = open(os.path.join(csrc, f)).read()
            if "__global__" in text or "__device__" in text:
                device.add(os.path.join("io_aware_exact_08_amd", "csrc", f))
    assert device and device <= set(bench.KERNEL_SOURCES)
