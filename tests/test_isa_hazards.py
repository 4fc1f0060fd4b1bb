"""Inline-asm MFMAs are invisible to the compiler's hazard recognizer.

Several kernels issue MFMAs from inline asm, to pin their accumulators to one
register file.  The compiler then inserts no wait states between a VALU write
of a VGPR and such an MFMA reading it, so the MFMA may read the old value.
The kernels are written so that only LDS/global loads (ordered by s_waitcnt)
write those operands.  This test compiles the device code and checks that no
VALU instruction writes a register that an inline-asm MFMA reads within the
next 12 instructions.  CPU only: hipcc cross-compiles for gfx950.
"""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_decoupled_rope_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SOURCES = ["attn_bf16.hip", "mha.hip"]


def _regs(spec):
    m = re.match(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


def _hazards(asm_text):
    """(kernel, valu, mfma) triples: a VALU write read by an inline-asm MFMA within 12 instructions."""
    found = []
    for name in re.findall(r"^(_Z\S*):", asm_text, re.M):
        start = asm_text.index(name + ":")
        end = asm_text.index(".Lfunc_end", start)
        body, in_asm = [], False
        for line in asm_text[start:end].split("\n"):
            t = line.strip()
            if "ASMSTART" in t:
                in_asm = True
                continue
            if "ASMEND" in t:
                in_asm = False
                continue
            if not t or t.startswith(";") or t.endswith(":") or t.startswith("."):
                continue
            body.append((t, in_asm))
        for i, (t, asm) in enumerate(body):
            op = t.split()[0]
            if asm or not op.startswith("v_") or op.startswith(("v_mfma", "v_accvgpr_read", "v_readlane",
                                                                  "v_readfirstlane", "v_cmp")):
                continue
            parts = t.split()
            written = _regs(parts[1].rstrip(",")) if len(parts) > 1 else set()
            if not written:
                continue
            for j in range(i + 1, min(i + 13, len(body))):
                tj, aj = body[j]
                if aj and tj.startswith("v_mfma"):
                    ops = [x.rstrip(",") for x in tj.split()[1:5]]
                    if written & (_regs(ops[1]) | _regs(ops[2]) | _regs(ops[3])):
                        found.append((name[:60], t, tj))
                        break
    return found


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", SOURCES)
def test_no_valu_write_feeds_inline_asm_mfma(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-Wno-unused-command-line-argument", "-o", str(out), os.path.join(CSRC, src)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    text = out.read_text()
    assert "v_mfma" in text
    assert _hazards(text) == []
