"""The bias kernels (d = 64, 128) and the 16-query-wave forward (d = 256 and
non-causal bf16 d = 128) issue the direct loads of their key or query loop as inline
assembly and count the waits themselves.  The compiler does not see those
loads, so any vmcnt wait it inserted inside the loop would miscount them (and
a vmcnt(0) would drain the whole pipeline).  Compile the d = 64 forward and
backward slices and the d = 256 (plain, split-KV) and d = 128 forward slices
to assembly and check that no compiler-inserted vmcnt wait appears at or after
the first loop header of any such kernel.  Waits written in the sources sit
between the assembler's inline-asm markers and are skipped."""
import os
import re
import subprocess

import pytest

from io_aware_exact_08_amd import build

BIAS_KERNEL = re.compile(r"^(_ZN2fa\d+(?:fwd_kernel|bwd_dkdv_kernel|bwd_dq_kernel)I\S*ELb1EEEvNS_7[FB]wdArgsE):")
Q16_KERNEL = re.compile(r"^(_ZN2fa14fwd_q16_kernelI\S*EEvNS_7FwdArgsE):")


def compiler_waits_in_loop(asm_text, kernel=BIAS_KERNEL):
    """{kernel: [compiler-inserted vmcnt waits at or after its first loop header]}."""
    out, cur, in_loop, in_asm = {}, None, False, False
    for line in asm_text.splitlines():
        m = kernel.match(line)
        if m:
            cur, in_loop, in_asm = m.group(1), False, False
            out[cur] = []
            continue
        if cur is None:
            continue
        if "s_endpgm" in line:
            cur = None
            continue
        if "Loop Header" in line:
            in_loop = True
        if ";;#ASMSTART" in line:
            in_asm = True
        elif ";;#ASMEND" in line:
            in_asm = False
        elif in_loop and not in_asm and re.search(r"s_waitcnt\b.*vmcnt", line):
            out[cur].append(line.strip())
    return out


def test_detector_on_a_sample():
    text = """_ZN2fa13bwd_dq_kernelILi64ELb0ELb0ELb1EEEvNS_7BwdArgsE:
\ts_waitcnt vmcnt(0)
.LBB0_1: ; =>This Inner Loop Header: Depth=1
\t;;#ASMSTART
\ts_waitcnt vmcnt(4)
\t;;#ASMEND
\ts_waitcnt vmcnt(1) lgkmcnt(0)
\ts_endpgm
"""
    assert compiler_waits_in_loop(text) == {
        "_ZN2fa13bwd_dq_kernelILi64ELb0ELb0ELb1EEEvNS_7BwdArgsE": ["s_waitcnt vmcnt(1) lgkmcnt(0)"]}


# (the plain d = 128 slice holds the two non-causal bf16 16-query kernels;
# causal bf16 runs fwd_kernel there)
@pytest.mark.parametrize("src,extra,kernel,count", [
    ("fa_fwd_inst.hip", ["-DFA_INST_D=64", "-DFA_INST_KIND=1"], BIAS_KERNEL, 4),
    ("fa_bwd_inst.hip", ["-DFA_INST_D=64"], BIAS_KERNEL, 4),
    ("fa_fwd_inst.hip", ["-DFA_INST_D=256", "-DFA_INST_KIND=0"], Q16_KERNEL, 4),
    ("fa_fwd_inst.hip", ["-DFA_INST_D=256", "-DFA_INST_KIND=2"], Q16_KERNEL, 4),
    ("fa_fwd_inst.hip", ["-DFA_INST_D=128", "-DFA_INST_KIND=0"], Q16_KERNEL, 2),
    ("fa_fwd_inst.hip", ["-DFA_INST_D=128", "-DFA_INST_KIND=2"], Q16_KERNEL, 2)])
def test_counted_loops_have_no_compiler_vmcnt_waits(tmp_path, src, extra, kernel, count):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not installed")
    out = str(tmp_path / "k.s")
    cmd = [hipcc] + build.HIPCC_FLAGS + extra + [
        "-I", os.path.join(build.ROOT, "include"), "--cuda-device-only", "-S",
        os.path.join(build.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        found = compiler_waits_in_loop(f.read(), kernel)
    assert len(found) >= count, sorted(found)
    bad = {k: v for k, v in found.items() if v}
    assert not bad, bad
