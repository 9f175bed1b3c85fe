"""The router's register-broadcast gate product issues v_fmac_f32_dpp from
inline asm, where the compiler inserts no wait states. The ISA requires two
wait states between a VALU instruction that writes a VGPR and a DPP
instruction that reads it; the kernel relies on the weight registers coming
straight from memory loads. This test compiles route.hip for gfx950 with the
library's flags and checks every v_fmac_f32_dpp in the generated assembly:
no VALU write of its DPP source register within the two preceding
instructions (s_nop n counts n + 1 wait states). CPU only: hipcc
cross-compiles."""
import os
import re
import shutil
import subprocess

import pytest

from mixture_experts_ffn_02_amd import build as B


def vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def hazards(asm_text):
    ins = []
    for line in asm_text.split("\n"):
        t = line.strip()
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        ins.append(t)
    found, n = [], 0
    for i, t in enumerate(ins):
        if not t.startswith("v_fmac_f32_dpp"):
            continue
        n += 1
        src = vregs(t.replace(",", " ").split()[2])
        waits = 0
        for j in range(i - 1, max(-1, i - 8), -1):
            p = ins[j]
            if p.startswith("s_nop"):
                waits += int(p.split()[1]) + 1
            else:
                if p.startswith("v_") and vregs(p.replace(",", " ").split()[1]) & src:
                    found.append((p, t))
                    break
                waits += 1
            if waits >= 2:
                break
    return n, found


def test_hazard_check_catches_a_planted_write():
    asm = "v_mov_b32_e32 v18, v3\nv_fmac_f32_dpp v58, v18, v34 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
    assert hazards(asm)[1]
    ok = "v_mov_b32_e32 v18, v3\ns_nop 1\nv_fmac_f32_dpp v58, v18, v34 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
    assert not hazards(ok)[1]


@pytest.mark.skipif(not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC), reason="hipcc not available")
def test_router_dpp_fmac_has_no_valu_hazard(tmp_path):
    out = tmp_path / "route.s"
    cmd = [B.HIPCC, *B.COMMON, *B.PER_FILE.get("route.hip", []), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "route.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    n, found = hazards(out.read_text())
    assert n > 0, "no v_fmac_f32_dpp in the router"
    assert not found, f"VALU write before a DPP read: {found[:3]}"
