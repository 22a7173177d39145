"""Build libflash_attn.so in-tree with hipcc for gfx950.

Each translation unit (the forward's instantiations in nine slices) compiles
to its own object in parallel, then one link.  The compiler's per-kernel
resource report (VGPRs, AGPRs, spills, scratch, occupancy, LDS) is written to
kernel_resources.json beside this file, keyed by a digest of the sources and
flags it describes.
"""
from __future__ import annotations

import hashlib
import json
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libflash_attn.so")
OBJDIR = os.path.join(ROOT, "_build")
RESOURCES = os.path.join(PKG, "kernel_resources.json")

# The d=256 backward keeps its dK/dV (and dQ) accumulators, 256 (128)
# registers per lane, in the accumulation registers: it is compiled without
# the flag that restricts MFMA accumulators to the ordinary VGPRs.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]

# (object name, source, extra defines, flags removed for this unit)
UNITS = [("flash_attn_api", "flash_attn_api.hip", [], []),
         ("fa_fwd", "fa_fwd.hip", [], []),
         ("fa_bwd", "fa_bwd.hip", [], [])]
UNITS += [(f"fa_fwd_inst_{d}_{k}", "fa_fwd_inst.hip", [f"-DFA_INST_D={d}", f"-DFA_INST_KIND={k}"], [])
          for d in (64, 128, 256) for k in (0, 1, 2)]
UNITS += [(f"fa_bwd_inst_{d}", "fa_bwd_inst.hip", [f"-DFA_INST_D={d}"], VGPR_FORM if d == 256 else [])
          for d in (64, 128, 256)]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler away from packed fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # MFMA accumulators in VGPRs (no AGPR copies around the softmax)
    *VGPR_FORM,
    # no NaN canonicalisation in max (infinities are still honoured)
    "-fno-honor-nans",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources_digest(extra_flags=()) -> str:
    """Digest of every kernel source, the public header and the compile flags."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp")))
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "include", "flash_attn.h"), "rb") as fh:
        h.update(fh.read())
    h.update(" ".join(HIPCC_FLAGS + list(extra_flags)).encode())
    return h.hexdigest()[:16]


_FIELDS = {
    "VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
    "Occupancy [waves/SIMD]": "occupancy_waves_per_simd", "SGPRs Spill": "sgpr_spill",
    "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds_bytes", "TotalSGPRs": "sgpr",
}


def parse_resource_remarks(text: str) -> dict:
    """kernel-resource-usage remarks -> {mangled name: {field: int}}."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([^:]+(?:\[[^\]]*\])?): (\S+) \[-Rpass-analysis", line)
        if m and cur is not None and m.group(1).strip() in _FIELDS:
            val = m.group(2)
            cur[_FIELDS[m.group(1).strip()]] = int(val) if val.lstrip("-").isdigit() else val
    return out


def demangle(names):
    tool = shutil.which("c++filt")
    if not tool or not names:
        return {n: n for n in names}
    res = subprocess.run([tool], input="\n".join(names), capture_output=True, text=True)
    dem = res.stdout.splitlines()
    return dict(zip(names, dem)) if len(dem) == len(names) else {n: n for n in names}


def _remove(flags, drop):
    """flags without the consecutive sequence `drop` (if present)."""
    n = len(drop)
    for i in range(len(flags) - n + 1):
        if n and flags[i:i + n] == drop:
            return flags[:i] + flags[i + n:]
    return list(flags)


def _compile(unit, extra_flags, verbose):
    name, src, defs, drop = unit
    obj = os.path.join(OBJDIR, name + ".o")
    cmd = [hipcc()] + _remove(HIPCC_FLAGS, drop) + list(extra_flags) + defs + \
        ["-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"),
         "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    text = res.stdout + res.stderr
    if res.returncode != 0:
        errs = "\n".join(l for l in text.splitlines()
                         if "packed-fp32-ops" not in l and "remark:" not in l)
        raise RuntimeError(f"hipcc failed on {src} {' '.join(defs)} ({res.returncode}):\n{errs}")
    return obj, parse_resource_remarks(text)


def build(verbose: bool = False, extra_flags=None, jobs: int | None = None) -> str:
    """Compile every HIP source and link one shared library; returns its path."""
    extra_flags = list(extra_flags or [])
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(UNITS), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda u: _compile(u, extra_flags, verbose), UNITS))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for o, _ in results] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    kernels = {}
    for _, rep in results:
        kernels.update(rep)
    names = demangle(sorted(kernels))
    rec = {"sources_sha256_16": sources_digest(extra_flags),
           "flags": HIPCC_FLAGS + extra_flags,
           "kernels": {names[k]: kernels[k] for k in sorted(kernels, key=lambda k: names[k])}}
    # the tracked summary describes the shipped flags only; other flags write
    # theirs beside their objects
    out = RESOURCES if not extra_flags else os.path.join(OBJDIR, "kernel_resources.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=False)
        f.write("\n")
    if verbose:
        spills = [(n, r) for n, r in rec["kernels"].items()
                  if r.get("vgpr_spill", 0) or r.get("sgpr_spill", 0) or r.get("scratch_bytes_per_lane", 0)]
        print(f"{len(rec['kernels'])} kernels; {len(spills)} with spills or scratch", flush=True)
        for n, r in spills:
            print(f"  {n}: vgpr_spill={r.get('vgpr_spill')} scratch={r.get('scratch_bytes_per_lane')}")
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
