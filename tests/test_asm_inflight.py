"""The generated gfx950 assembly of the attention kernels never touches a
register that an in-flight LDS read will still write.

The kernels read LDS operands with inline-asm ds_read_b128 /
ds_read_b64_tr_b16 and wait for them with explicit s_waitcnt lgkmcnt(N)
statements tied to the result registers.  The compiler takes an asm
statement's outputs as written when the statement issues, so under register
pressure it may copy such a result (to an AGPR, to scratch) or hand its
register to another value before the wait: the copy then holds stale data
and the late-arriving read overwrites whatever took the register.  This test
compiles every attention translation unit to assembly with the library's own
flags and walks each kernel in order, retiring outstanding LDS operations at
each s_waitcnt lgkmcnt(N) (they complete in issue order), and fails on any
instruction that names a register an outstanding read still targets.

CPU only: hipcc cross-compiles gfx950 here.
"""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from attention_fa2_tiles_amd import build

AUDITED = ("attn_fwd.hip", "attn_bwd.hip", "attn_fwd_fp8.hip")
_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")
_ASM_READS = ("ds_read_b128", "ds_read_b64_tr_b16")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), r) for r in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def inflight_conflicts(asm):
    """{kernel symbol: [offending instructions]} for an assembly listing."""
    found = {}
    for m in re.finditer(r"^(_Z[^:\s]*):", asm, re.M):
        name = m.group(1)
        end = asm.find("; -- End function", m.start())
        pending = []   # destination registers of LDS operations in issue order (None: no result)
        bad = []
        for line in asm[m.start():end].split("\n"):
            t = line.split(";")[0].strip()
            if not t or t.endswith(":") or t.startswith("."):
                continue
            op = t.split()[0]
            operands = t[len(op):]
            if op == "s_waitcnt":
                w = re.search(r"lgkmcnt\((\d+)\)", t)
                if w:
                    n = int(w.group(1))
                    pending = pending[len(pending) - n:] if 0 < n < len(pending) else ([] if n == 0 else pending)
                continue
            live = set().union(*[d for d in pending if d]) if pending else set()
            dest = _regs(operands.split(",")[0])
            if op.startswith(_ASM_READS):
                if dest & live:
                    bad.append(t)
            elif _regs(operands) & live:
                bad.append(t)
            if op.startswith("ds_"):
                pending.append(dest if op.startswith("ds_read") else None)
        if bad:
            found[name] = bad
    return found


def test_checker_flags_a_copy_of_an_inflight_result():
    """The walk itself: a copy of a read's destination before its wait, and
    a reuse of that register, are flagged; the same code with the wait first
    is not."""
    bad = """_Zkern:
    ds_read_b128 v[4:7], v1 offset:0
    ds_read_b128 v[8:11], v1 offset:64
    v_accvgpr_write_b32 a0, v5
    s_waitcnt lgkmcnt(1)
    v_mfma_f32_32x32x16_bf16 v[12:27], v[4:7], v[30:33], 0
    v_mov_b32 v9, 0
    s_waitcnt lgkmcnt(0)
; -- End function
"""
    good = bad.replace("    v_accvgpr_write_b32 a0, v5\n    s_waitcnt lgkmcnt(1)\n",
                       "    s_waitcnt lgkmcnt(1)\n    v_accvgpr_write_b32 a0, v5\n")
    good = good.replace("    v_mov_b32 v9, 0\n    s_waitcnt lgkmcnt(0)\n", "    s_waitcnt lgkmcnt(0)\n    v_mov_b32 v9, 0\n")
    got = inflight_conflicts(bad)["_Zkern"]
    assert got == ["v_accvgpr_write_b32 a0, v5", "v_mov_b32 v9, 0"], got
    assert inflight_conflicts(good) == {}


def _compile_asm(unit, out_dir):
    src, extra, name = unit
    out = os.path.join(out_dir, name + ".s")
    cmd = [build.hipcc()] + build.compile_flags() + extra + [
        "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return name, out


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_register_touched_while_lds_read_in_flight(tmp_path):
    units = [u for u in build.units() if u[0] in AUDITED]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        outs = list(ex.map(lambda u: _compile_asm(u, str(tmp_path)), units))
    problems = {}
    for name, path in outs:
        with open(path) as f:
            for kern, bad in inflight_conflicts(f.read()).items():
                problems[f"{name}: {kern}"] = bad[:4]
    assert not problems, "registers touched while an LDS read is in flight:\n" + "\n".join(
        f"{k}\n    " + "\n    ".join(v) for k, v in problems.items())
