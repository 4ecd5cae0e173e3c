"""Static check of the generated gfx950 assembly (CPU only: hipcc cross-compiles).

A load written in inline assembly is invisible to the compiler's wait-count tracking: the
compiler takes its destination registers as written when the asm statement ends. If the
statement does not itself wait for the load, a register copy, spill or other read that the
compiler places before the explicit wait would take stale data, and whether it does depends on
register allocation. The kernels keep every such load safe by waiting inside the same asm
statement (the decode kernel's page-id reload) or by loading through LDS (the K/V and Q rings).
This test compiles the kernels with the library's flags and scans the assembly. It counts the
inline-asm loads into VGPRs whose asm block ends before a wait retires them ("deferred" loads),
and requires that there are none. The scan itself (registers touched between such a load and
the ``s_waitcnt vmcnt(N)`` that provably retires it, N not above the number of later loads) is
pinned on hand-written assembly. The scan is linear, so it follows the fall-through path of each
branch.
"""
import os
import re
import shutil
import subprocess

import pytest

from gqa_attention_sinks_sink_amd import build

CSRC = os.path.join(build.ROOT, "gqa_attention_sinks_sink_amd", "csrc")
VMEM_LOAD = re.compile(r"^(buffer_load|global_load|scratch_load|flat_load)")


def _regs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def scan(lines):
    """(deferred loads, list of violations) for one function's assembly lines. A deferred load is an
    inline-asm load into VGPRs still outstanding when its asm block ends."""
    pending = []  # [registers, loads issued after it, line number]
    deferred, bad = 0, []
    in_asm = False
    block = []  # pending entries created in the current asm block
    for n, raw in enumerate(lines, 1):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            block = []
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            deferred += sum(1 for e in block if any(e is p for p in pending))
            continue
        s = s.split(";")[0].strip()
        if not s or s.endswith(":") or s.startswith("."):
            continue
        op = s.split()[0]
        toks = [t for t in re.split(r"[ ,]+", s)[1:] if t]
        if op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", s)
            if m:
                lim = int(m.group(1))
                pending = [p for p in pending if p[1] < lim]
            continue
        untracked = in_asm and VMEM_LOAD.match(op) and " lds" not in f" {s} " and toks and toks[0].startswith("v")
        used = set()
        for t in toks[1:] if untracked else toks:  # an untracked load's own destination is no use
            used |= _regs(t)
        for regs, _, at in pending:
            if used & regs:
                bad.append(f"line {n}: '{s}' touches v{sorted(used & regs)} loaded at line {at}")
        if VMEM_LOAD.match(op):
            for p in pending:
                p[1] += 1
        if untracked:
            entry = [_regs(toks[0]), 0, n]
            pending.append(entry)
            block.append(entry)
    return deferred, bad


def kernel_bodies(asm):
    lines = asm.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_ZN9attn_sink\w+:", l)]
    for s in starts:
        e = next(i for i in range(s, len(lines)) if lines[i].startswith(".Lfunc_end"))
        yield lines[s].split(":")[0], lines[s:e]


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", ["decode.hip", "prefill.hip", "rope.hip", "merge.hip"])
def test_no_inline_asm_load_outlives_its_asm_block(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [build.hipcc(), *build.compile_flags(), "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    problems = []
    for name, body in kernel_bodies(out.read_text()):
        deferred, bad = scan(body)
        if deferred:
            problems.append(f"{name}: {deferred} inline-asm VGPR load(s) not retired inside their asm block")
        problems += [f"{name}: {b}" for b in bad[:3]]
    assert not problems, "\n".join(problems)


def test_scan_flags_a_copy_before_the_wait():
    asm = """
	;;#ASMSTART
	global_load_dwordx4 v[2:5], v[8:9], off
	;;#ASMEND
	buffer_load_dwordx4 v[10:13], v1, s[0:3], 0 offen
	v_mov_b32_e32 v20, v3
	s_waitcnt vmcnt(2)
	v_mov_b32_e32 v21, v4
	s_waitcnt vmcnt(1)
	v_mov_b32_e32 v22, v5
""".split("\n")
    deferred, bad = scan(asm)
    assert deferred == 1
    # flagged: the copy before any wait, and the one after vmcnt(2) (one later load: the untracked
    # one may still be in flight); vmcnt(1) retires it
    assert len(bad) == 2 and "v20" in bad[0] and "v21" in bad[1]


def test_scan_accepts_a_load_retired_in_its_own_block():
    asm = """
	;;#ASMSTART
	global_load_dword v7, v[8:9], off
	s_waitcnt vmcnt(0)
	;;#ASMEND
	v_readlane_b32 s4, v7, 3
	;;#ASMSTART
	buffer_load_dwordx4 v1, s[0:3], 0 offen lds
	;;#ASMEND
""".split("\n")
    deferred, bad = scan(asm)
    assert deferred == 0 and not bad
