"""Static check of the gfx950 code of the decode kernels: every DPP read
(the row broadcasts written as inline assembly in quant.hpp and
experts_decode.hip, and the compiler's own DPP moves) must see its source
VGPR at least 2 wait states after the last VALU write of it, and no VALU
write of EXEC may come within 5 wait states of a DPP instruction (the DPP
hazards of the CDNA instruction set).  The compiler's hazard recognizer
does not look inside inline assembly, so this test recompiles the sources
to assembly and scans them."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_routed_expert_router_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")

DPP_MARKS = ("_dpp", "row_newbcast", "quad_perm", "row_shr", "row_shl", "row_mirror",
             "row_half_mirror", "row_bcast")


def _vregs(tok):
    tok = tok.strip().rstrip(",")
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def dpp_hazards(asm_text):
    """List of (line number, problem, instruction, earlier instruction)."""
    found = []
    hist = []   # (is_valu, vgpr dsts, writes exec, wait states, text, is label)
    for ln, raw in enumerate(asm_text.splitlines(), 1):
        s = raw.split(";")[0].strip()
        if not s or (s.startswith(".") and not s.endswith(":")):
            continue
        if s.endswith(":"):
            hist.append((False, set(), False, 0, s, True))
            continue
        parts = s.replace(",", " ").split()
        op = parts[0]
        ws = int(parts[1], 0) + 1 if op == "s_nop" else 1
        valu = op.startswith("v_")
        writes_exec = valu and (op.startswith("v_cmpx") or (len(parts) > 1 and parts[1] == "exec"))
        vdst = set()
        if valu and not op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")) and len(parts) > 1:
            vdst = _vregs(parts[1])
        if any(mk in s for mk in DPP_MARKS) and len(parts) > 2:
            src0 = _vregs(parts[2])
            acc = 0
            for h_valu, h_dst, h_exec, h_ws, h_text, h_label in reversed(hist):
                if h_label:
                    # a branch target inside the window: the other path must be
                    # checked too; demand a full window instead
                    if acc < 5:
                        found.append((ln, "branch target within 5 wait states", s, h_text))
                    break
                if acc < 2 and h_valu and (h_dst & src0):
                    found.append((ln, "VALU write of the DPP source", s, h_text))
                if acc < 5 and h_exec:
                    found.append((ln, "VALU write of EXEC", s, h_text))
                acc += h_ws
                if acc >= 5:
                    break
        hist.append((valu, vdst, writes_exec, ws, s, False))
        del hist[:-64]
    return found


def test_scanner_finds_a_planted_hazard():
    bad = "\tv_mad_u32_u24 v1, v0, 3, 1\n\tv_mov_b32_e32 v2, 0\n" \
          "\tv_dot8c_i32_i4_dpp v3, v1, v2 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
    assert len(dpp_hazards(bad)) == 1
    ok = "\tv_mad_u32_u24 v1, v0, 3, 1\n\ts_nop 1\n" \
         "\tv_dot8c_i32_i4_dpp v3, v1, v2 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
    assert dpp_hazards(ok) == []


@pytest.mark.parametrize("src", ["experts_decode.hip", "route_decode.hip", "route.hip"])
def test_no_dpp_hazards(src, tmp_path):
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "strata_build", os.path.join(ROOT, "quantized_routed_expert_router_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    flags = [f for f in b.HIP_FLAGS if f != "-fPIC"]
    out = tmp_path / (src + ".s")
    r = subprocess.run(["hipcc", *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src),
                        "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    assert "_dpp" in text or "row_" in text or "quad_perm" in text
    problems = dpp_hazards(text)
    assert problems == [], "\n".join(" | ".join(map(str, p)) for p in problems[:20])
