"""An LDS read whose array starts 64 KB or more into the workgroup's LDS cannot
fold the array's address into the instruction's 16-bit offset field.  Left to
itself the compiler then adds that address with a VALU op before every read
inside the key loop (the d = 256 forward's V stages start at 64 KB; the d = 64
bias forwards can place V there too).  Those kernels keep the address in the
per-lane read bases instead.  Compile their slices to assembly and check that
no loop adds a literal of 64 KB or more to a VGPR."""
import os
import re
import subprocess

import pytest

from io_aware_exact_08_amd import build

Q16_KERNEL = re.compile(r"^(_ZN2fa14fwd_q16_kernelI\S*EEvNS_7FwdArgsE):")
BIAS_FWD_KERNEL = re.compile(r"^(_ZN2fa10fwd_kernelI\S*ELb1EEEvNS_7FwdArgsE):")
BIG_ADD = re.compile(r"\bv_(?:or|add)_(?:b32|u32)_e32\s+v\d+,\s*0x([0-9a-fA-F]+),\s*v\d+")


def big_adds_in_loop(asm_text, kernel):
    """{kernel: [adds of an LDS-sized literal (64 KB up to 256 KB; gfx950 has
    160 KB) to a VGPR at or after its first loop header]}."""
    out, cur, in_loop = {}, None, False
    for line in asm_text.splitlines():
        m = kernel.match(line)
        if m:
            cur, in_loop = m.group(1), False
            out[cur] = []
            continue
        if cur is None:
            continue
        if "s_endpgm" in line:
            cur = None
            continue
        if "Loop Header" in line:
            in_loop = True
        m = BIG_ADD.search(line)
        if in_loop and m and 0x10000 <= int(m.group(1), 16) < 0x40000:
            out[cur].append(line.strip())
    return out


def test_detector_on_a_sample():
    text = """_ZN2fa14fwd_q16_kernelILi256ELb0ELb0ELb0ELb0EEEvNS_7FwdArgsE:
\tv_or_b32_e32 v1, 0x10000, v2
.LBB0_1: ; =>This Inner Loop Header: Depth=1
\tv_or_b32_e32 v3, 0x12000, v141
\tv_add_u32_e32 v4, 0x200, v5
\tv_add_u32_e32 v9, 0xffffff80, v5
\tds_read_b64_tr_b16 v[6:7], v8 offset:57344
\ts_endpgm
"""
    assert big_adds_in_loop(text, Q16_KERNEL) == {
        "_ZN2fa14fwd_q16_kernelILi256ELb0ELb0ELb0ELb0EEEvNS_7FwdArgsE": ["v_or_b32_e32 v3, 0x12000, v141"]}


@pytest.mark.parametrize("extra,kernel,count", [
    (["-DFA_INST_D=256", "-DFA_INST_KIND=0"], Q16_KERNEL, 6),
    (["-DFA_INST_D=256", "-DFA_INST_KIND=2"], Q16_KERNEL, 4),
    (["-DFA_INST_D=64", "-DFA_INST_KIND=1"], BIAS_FWD_KERNEL, 8)])
def test_loops_add_no_lds_array_base(tmp_path, extra, kernel, count):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not installed")
    out = str(tmp_path / "k.s")
    cmd = [hipcc] + build.HIPCC_FLAGS + extra + [
        "-I", os.path.join(build.ROOT, "include"), "--cuda-device-only", "-S",
        os.path.join(build.CSRC, "fa_fwd_inst.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        found = big_adds_in_loop(f.read(), kernel)
    assert len(found) >= count, sorted(found)
    assert all(not v for v in found.values()), {k: v[:3] for k, v in found.items() if v}
