"""Static check of the built gfx950 code for a hazard that the compiler does
not guard inside inline assembly (CPU only; disassembles the library built
here with the ROCm llvm-objdump).

gfx9 requires 5 wait states between a VALU instruction that writes an SGPR
(v_readfirstlane_b32, v_readlane_b32, a compare writing an SGPR pair) and a
buffer instruction that reads that SGPR as its resource or offset. The
compiler inserts them for the memory instructions it emits itself, but the
LDS-DMA loads are inline assembly, which its hazard checks do not inspect: a
resource rebuilt inside a pipeline must be settled before the asm reads it.
A violation lets the load see the SGPR's old value (a stale base address or
size), which shows up only now and then. This scans every buffer
instruction of every kernel in the library and also checks that each
LDS-DMA load has its M0 write and one wait state before it.
"""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "rollout_rlk_linear_amd", "librlk_linear.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
VALU_SGPR_WAIT = 5


def _sgprs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    if m:
        return {int(m.group(1))}
    if tok in ("vcc", "vcc_lo"):
        return {"vcc"}
    return set()


def scan(lines):
    """(hazards, buffer instructions seen, LDS-DMA loads without M0 setup)."""
    instrs = []
    func = None
    for line in lines:
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            func = m.group(1)
            instrs.append((func, None))
            continue
        t = line.split("//")[0].split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        instrs.append((func, t))
    hazards, nbuf, bad_m0 = [], 0, []
    for i, (f, t) in enumerate(instrs):
        if t is None or not t.startswith("buffer_"):
            continue
        nbuf += 1
        ops = t.split(None, 1)[1].split(",") if " " in t else []
        reads = set()
        for o in ops[1:]:
            for w in o.split():
                reads |= _sgprs(w)
        ws, j = 0, i - 1
        while j >= 0 and ws < VALU_SGPR_WAIT and instrs[j][1] is not None:
            u = instrs[j][1]
            m = re.match(r"s_nop (\d+)", u)
            if m:
                ws += int(m.group(1)) + 1
                j -= 1
                continue
            if u.startswith("v_"):
                dst = u.split(None, 1)[1].split(",")[0] if " " in u else ""
                w = _sgprs(dst)
                if u.startswith("v_cmp") and not w:
                    w = {"vcc"}
                if w & reads:
                    hazards.append(f"{f}: '{u}' {ws} wait states before '{t}'")
            ws += 1
            j -= 1
        if t.endswith(" lds"):
            prev = [x[1] for x in instrs[max(0, i - 2):i]]
            if len(prev) < 2 or not prev[0].startswith("s_mov_b32 m0") or not prev[1].startswith("s_nop"):
                bad_m0.append(f"{f}: {prev} before '{t}'")
    return hazards, nbuf, bad_m0


def test_scanner_finds_a_planted_hazard():
    planted = """0000000000001000 <k>:
	v_readfirstlane_b32 s18, v53
	v_cndmask_b32_e64 v0, v53, v13, s[0:1]
	s_waitcnt lgkmcnt(0)
	buffer_store_dwordx4 v[118:121], v0, s[16:19], 0 offen nt
	s_mov_b32 m0, s2
	buffer_load_dwordx4 v1, s[4:7], s6 offen lds
""".splitlines()
    hz, nbuf, bad = scan(planted)
    assert nbuf == 2 and len(hz) == 1 and "s18" in hz[0] and len(bad) == 1
    settled = [l.replace("s_waitcnt lgkmcnt(0)", "s_nop 4") for l in planted]
    assert scan(settled)[0] == []


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="ROCm llvm-objdump not installed")
def test_built_library_has_no_valu_sgpr_buffer_hazard():
    if not os.path.exists(LIB):
        pytest.skip("library not built (__graft_entry__.build())")
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "lib.so")
        shutil.copy(LIB, so)
        subprocess.run([OBJDUMP, "--offloading", so], cwd=d, check=True, capture_output=True)
        objs = sorted(f for f in os.listdir(d) if "gfx950" in f)
        assert objs, "no gfx950 code objects in the library"
        total, hazards, bad_m0 = 0, [], []
        for o in objs:
            dis = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", os.path.join(d, o)],
                                 check=True, capture_output=True, text=True).stdout
            hz, nbuf, bad = scan(dis.splitlines())
            total += nbuf
            hazards += hz
            bad_m0 += bad
    assert total > 100, f"only {total} buffer instructions found"
    assert not hazards, "\n".join(hazards[:20])
    assert not bad_m0, "\n".join(bad_m0[:20])
