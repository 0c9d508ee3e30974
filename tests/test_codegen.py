"""Code-generation checks on the gfx950 assembly of the kernels (CPU only).

An MFMA executes for all 64 lanes whatever the EXEC mask says, so an MFMA
that the compiler places inside an EXEC-masked region (s_and_saveexec ...
s_or exec) with no s_cbranch_execz skip computes even when its guarding
condition is false. The kernels keep every MFMA guard wave-uniform (scalar
branch); this test fails if the compiler ever emits the masked form.
It also checks that no packed-fp32 VALU instruction is emitted.
"""
import os
import re
import shutil
import subprocess

import pytest

from kimi_delta_attention_03_amd import build as kbuild

HIP_SOURCES = [s for s in kbuild.SOURCES if s.endswith(".hip")]


def _asm(src, tmp_path):
    hipcc = kbuild.hipcc()
    out = tmp_path / (src + ".s")
    cmd = [hipcc, *kbuild.FLAGS, "--cuda-device-only", "-S", os.path.join(kbuild.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


def masked_mfma_count(asm: str) -> int:
    """MFMAs on the fall-through path of an EXEC-masked region with no
    s_cbranch_execz skip. An unconditional s_branch ends the fall-through path:
    the code after it is another block, entered only by jumps (a masked body
    that the compiler moved elsewhere is scanned at its own place, after its
    own s_and_saveexec)."""
    bad, in_mask, skipped = 0, False, False
    for line in asm.splitlines():
        t = line.strip()
        if t.startswith("s_and_saveexec") or t.startswith("s_andn2_saveexec"):
            in_mask, skipped = True, False
        elif in_mask and t.startswith("s_cbranch_execz"):
            skipped = True
        elif in_mask and (re.match(r"s_(or|mov)_b64\s+exec", t) or re.match(r"s_branch\s", t)):
            in_mask = False
        elif in_mask and not skipped and t.startswith("v_mfma"):
            bad += 1
    return bad


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_exec_masked_mfma_and_no_packed_fp32(src, tmp_path):
    asm = _asm(src, tmp_path)
    assert masked_mfma_count(asm) == 0
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", asm)


def test_detector_flags_masked_mfma():
    snippet = """
    s_and_saveexec_b64 s[2:3], vcc
    v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]
    s_or_b64 exec, exec, s[2:3]
    """
    assert masked_mfma_count(snippet) == 1
    skipped = snippet.replace("vcc\n", "vcc\n    s_cbranch_execz .L1\n")
    assert masked_mfma_count(skipped) == 0
    # a masked store block placed out of line, jumping back into its body; the
    # block after the unconditional branch is entered by a scalar branch
    out_of_line = """
    s_and_saveexec_b64 s[0:1], s[2:3]
    s_cbranch_execnz .L37
    s_branch .L38
.L81:
    v_mfma_f32_16x16x4_f32 v[0:3], v28, v33, v[0:3]
    """
    assert masked_mfma_count(out_of_line) == 0
    # an MFMA before the branch is still on the masked path
    before = out_of_line.replace("    s_cbranch_execnz .L37\n",
                                 "    v_mfma_f32_16x16x4_f32 v[0:3], v28, v33, v[0:3]\n    s_cbranch_execnz .L37\n")
    assert masked_mfma_count(before) == 1
