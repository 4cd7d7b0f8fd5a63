"""Wait states in the gfx950 code (CPU only: the kernels are compiled to assembly).

A vector memory instruction that reads an SGPR written by a VALU instruction
needs five wait states on this architecture.  The compiler pads its own
instructions for that hazard but not inline assembly, and the direct-to-LDS
loads are inline assembly whose base address the compiler often writes with
v_readfirstlane just before.  Every vector memory instruction of every kernel
must have at least five wait states (instructions, or s_nop n counting n + 1)
between it and the last VALU write of any SGPR it reads; a direct-to-LDS load
must have them inside its own basic block."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["mla_decode.hip", "mla_prefill.hip", "mla_gemm.hip", "mla_append.hip"]
VMEM = ("global_", "buffer_", "scratch_", "flat_")
NEEDED = 5


def _sgprs(text):
    regs = set()
    for a, b in re.findall(r"\bs\[(\d+):(\d+)\]", text):
        regs |= {f"s{k}" for k in range(int(a), int(b) + 1)}
    regs |= set(re.findall(r"\b(s\d+)\b", text))
    return regs


def _violations(asm: str):
    """(instruction, wait states found) for each vector memory instruction with
    fewer than NEEDED wait states after a VALU write of one of its SGPRs."""
    out, block = [], []
    for raw in asm.splitlines():
        line = raw.split(";")[0].rstrip()
        if not line.strip() or line.strip().startswith("."):
            continue
        if not raw.startswith("\t"):  # a label: a new basic block
            block = []
            continue
        ins = line.strip()
        op = ins.split()[0]
        if op.startswith(VMEM):
            used = _sgprs(ins.split(None, 1)[1]) if " " in ins else set()
            if used:
                ws, found = 0, False
                for prev in reversed(block):
                    if ws >= NEEDED:
                        found = True
                        break
                    pop = prev.split()[0]
                    if pop.startswith("s_nop"):
                        ws += int(prev.split()[1], 0) + 1
                        continue
                    dst = prev.split()[1].rstrip(",") if len(prev.split()) > 1 else ""
                    if pop.startswith("v_") and _sgprs(dst) & used:
                        out.append((ins, ws))
                        found = True
                        break
                    ws += 1
                if not found and ws < NEEDED and "_lds_" in op:
                    out.append((ins, ws))  # the block starts too close to a direct-to-LDS load
        block.append(ins)
    return out


def _compile(src, tmp):
    from mla_attention_paged_amd import _build
    out = os.path.join(tmp, src + ".s")
    cmd = [_build.hipcc()] + _build.flags() + ["-x", "hip", "--cuda-device-only", "-S",
                                               os.path.join(_build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_vmem_sgpr_wait_states(tmp_path):
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        asms = list(ex.map(lambda s: _compile(s, str(tmp_path)), SOURCES))
    dma = 0
    for src, asm in zip(SOURCES, asms):
        dma += asm.count("global_load_lds_dwordx4")
        bad = _violations(asm)
        assert not bad, f"{src}: {len(bad)} vector memory instructions too close to a VALU SGPR write: {bad[:4]}"
    assert dma > 0


def test_scanner_finds_the_hazard():
    """The scanner itself: a load right behind v_readfirstlane of its base fails,
    the padded form passes."""
    bad = "f:\n\tv_readfirstlane_b32 s10, v6\n\ts_mov_b32 m0, s4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v1, s[10:11]\n"
    good = ("f:\n\tv_readfirstlane_b32 s10, v6\n\ts_nop 2\n\ts_mov_b32 m0, s4\n\ts_nop 0\n"
            "\tglobal_load_lds_dwordx4 v1, s[10:11]\n")
    top = "f:\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v1, s[10:11]\n"
    assert _violations(bad) == [("global_load_lds_dwordx4 v1, s[10:11]", 2)]
    assert _violations(good) == []
    assert len(_violations(top)) == 1
