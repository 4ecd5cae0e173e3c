"""Static check of the generated gfx950 assembly (CPU only: hipcc cross-compiles).

The decode kernel loads Q into registers with inline-assembly loads that the compiler does not
track, so that waiting for them does not also wait for the K/V loads issued after them. That is
only correct while no instruction reads or moves those registers before an explicit wait has
retired the load: the compiler believes the value is there as soon as the asm statement ends,
and a register copy or spill placed before the wait would take stale data. Whether it does so
depends on register allocation, so this test compiles the kernels with the library's flags and
scans the assembly: after each untracked load into VGPRs, every instruction up to the
``s_waitcnt vmcnt(N)`` that provably retires it (N not above the number of later loads, which
return in order) must leave its destination registers alone. The scan is linear, so it follows
the fall-through path of each branch.
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
    """(untracked loads seen, list of violations) for one function's assembly lines."""
    pending = []  # [registers, loads issued after it, line number]
    seen, bad = 0, []
    in_asm = False
    for n, raw in enumerate(lines, 1):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
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
            pending.append([_regs(toks[0]), 0, n])
            seen += 1
    return seen, bad


def kernel_bodies(asm):
    lines = asm.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_ZN9attn_sink\w+:", l)]
    for s in starts:
        e = next(i for i in range(s, len(lines)) if lines[i].startswith(".Lfunc_end"))
        yield lines[s].split(":")[0], lines[s:e]


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", ["decode.hip", "prefill.hip", "rope.hip", "merge.hip"])
def test_untracked_register_loads_are_not_touched_before_their_wait(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [build.hipcc(), *build.compile_flags(), "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    total_seen, problems = 0, []
    for name, body in kernel_bodies(out.read_text()):
        seen, bad = scan(body)
        total_seen += seen
        problems += [f"{name}: {b}" for b in bad[:3]]
    assert not problems, "\n".join(problems)
    if src == "decode.hip":
        assert total_seen > 0, "the decode kernel's untracked Q loads were not found (scan inactive)"


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
    seen, bad = scan(asm)
    assert seen == 1
    # flagged: the copy before any wait, and the one after vmcnt(2) (one later load: the untracked
    # one may still be in flight); vmcnt(1) retires it
    assert len(bad) == 2 and "v20" in bad[0] and "v21" in bad[1]
