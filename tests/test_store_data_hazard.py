"""A CPU check of the library's gfx950 code: no vector store of more than
64 bits has its data registers overwritten by the very next instruction.

On gfx950 a 16-byte buffer or global store reads its data registers after it
issues, so the next VALU instruction must not write them yet.  The compiler
guards buffer stores only when their soffset operand is not a register; a
GEMM2 epilogue that passed column offsets in soffset had the next
instruction's write reach the first stored dword (the y rows of d_model 16384
came out wrong in one float of every four).  The kernels now keep soffset at
0; this test compiles every HIP source of the library to assembly (no GPU
needed) and checks the rule on every such store.
"""

import os
import re
import subprocess
import tempfile

import pytest

from moe_expert_layer_sigmoid_amd import build as libbuild

pytestmark = pytest.mark.slow


def _regs(spec):
    m = re.match(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


def store_data_hazards(asm_lines):
    """(line, store, next instruction) for every wide store whose data
    registers the next instruction, a VALU op, writes."""
    found = []
    for i, line in enumerate(asm_lines):
        m = re.match(r"(buffer|global)_store_dword(x3|x4)\s+(\S+?),", line)
        if not m:
            continue
        data = m.group(3) if m.group(1) == "buffer" else line.split()[2].rstrip(",")
        j = i + 1
        while j < len(asm_lines) and (not asm_lines[j] or asm_lines[j][0] in ";."):
            j += 1
        nxt = asm_lines[j] if j < len(asm_lines) else ""
        if nxt.startswith("v_") and _regs(nxt.split()[1].rstrip(",")) & _regs(data):
            found.append((i, line, nxt))
    return found


def test_checker_finds_the_pattern():
    asm = ["buffer_store_dwordx4 v[20:23], v33, s[12:15], s74 offen", "v_fma_f32 v20, v190, v20, 0",
           "buffer_store_dwordx4 v[24:27], v33, s[12:15], 0 offen", "s_nop 0", "v_fma_f32 v24, v1, v24, 0",
           "global_store_dwordx4 v[2:3], v[8:11], off", "v_add_u32_e32 v9, 1, v9"]
    assert [h[0] for h in store_data_hazards(asm)] == [0, 5]


@pytest.mark.parametrize("src", libbuild.SOURCES)
def test_no_wide_store_data_hazard(src):
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, src + ".s")
        cmd = [libbuild.hipcc(), *libbuild.flags(), "-S", "--cuda-device-only",
               os.path.join(libbuild.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        lines = [l.strip() for l in open(out)]
    bad = store_data_hazards(lines)
    assert not bad, "\n".join(f"line {i}: {s}  next: {n}" for i, s, n in bad[:10])
