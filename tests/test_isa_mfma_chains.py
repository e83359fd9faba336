"""ISA check (CPU, needs hipcc): no MFMA takes as srcC the result of an MFMA
of a different shape issued shortly before it.

On gfx950 a 16x16x16 bf16 MFMA accumulating onto a 16x16x32 bf16 MFMA's
result still in flight read stale srcC registers (wrong rows of some chunks,
non-deterministically), so the prefill kernels never form such chains.  This
test compiles the prefill sources exactly as the library build does and scans
every kernel's ISA for one."""
import os
import re
import shutil
import subprocess

import pytest

from linear_attention_recurrence_05_amd import build as kbuild

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


def _regs(spec):
    m = re.match(r"([va])\[(\d+):(\d+)\]", spec)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", spec)
    return {spec} if m else set()


def mixed_shape_chains(asm_lines, window=12):
    """(writer index, reader index, writer op, reader op) for every MFMA whose
    srcC registers were last written by an MFMA of another opcode fewer than
    `window` instructions earlier."""
    last = {}
    found = []
    lines = [l.strip() for l in asm_lines if l.strip() and not l.strip().startswith((";", "."))]
    for i, l in enumerate(lines):
        parts = l.split(None, 1)
        if len(parts) < 2:
            continue
        op, ops = parts[0], [o.strip() for o in parts[1].split(",")]
        if op.startswith("v_mfma"):
            if len(ops) > 3:
                hits = {last[r] for r in _regs(ops[3])
                        if r in last and last[r][0] != op and i - last[r][1] < window}
                found.extend((wi, i, wop, op) for wop, wi in sorted(hits, key=lambda x: x[1]))
            for r in _regs(ops[0]):
                last[r] = (op, i)
        elif ops:
            for r in _regs(ops[0]):
                last.pop(r, None)
    return found


def test_scanner_flags_a_planted_chain():
    asm = ["v_mfma_f32_16x16x32_bf16 a[32:35], v[0:3], v[8:11], a[32:35]",
           "v_mfma_f32_16x16x16_bf16 a[32:35], v[198:199], v[30:31], a[32:35]"]
    assert len(mixed_shape_chains(asm)) == 1
    same = ["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
            "v_mfma_f32_16x16x32_bf16 v[0:3], v[12:15], v[16:19], v[0:3]"]
    assert mixed_shape_chains(same) == []


@pytest.mark.parametrize("source", ["kda_prefill.hip", "kda_pair.hip", "kda_bwd_chunk.hip"])
def test_prefill_kernels_have_no_mixed_shape_srcc_chain(tmp_path, source):
    # the flags the library build gives this source, device-only assembly
    hipcc = os.environ.get("HIPCC", "hipcc")
    src = os.path.join(kbuild.CSRC, source)
    asm = tmp_path / "prefill.s"
    subprocess.run([hipcc, *kbuild.source_flags(source), "--cuda-device-only", "-S", src, "-o", str(asm)],
                   check=True, capture_output=True)
    text = asm.read_text().split("\n")
    assert any("v_mfma_f32_16x16x32_bf16" in l for l in text)
    assert mixed_shape_chains(text) == []
