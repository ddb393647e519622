"""Machine-code check of the built kernels (CPU only): the transposing LDS
reads are issued as inline assembly (ds_read_b64_tr_b16), whose result the
compiler believes is written at once.  If register allocation copies,
reuses or spills a destination register of such a read before the wave has
waited for it (s_waitcnt lgkmcnt(0)), the kernel computes with stale or
clobbered values, and a clobbered address register can make a later load
or store fault.  This test disassembles the gfx950 code objects of every
built object file and walks every control-flow path from each such read to
its wait: no instruction on the way may read or write the read's
destination registers."""
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "dense_gemm_12_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

_INSN = re.compile(r"^\s+([a-z_0-9]+)(?:\s+([^/]*?))?\s*//\s*([0-9A-Fa-f]+):")
_FUNC = re.compile(r"^([0-9a-f]+) <([^>]+)>:")


def _regs(ops):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", ops or ""):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _disassemble(obj, tmp):
    fb = os.path.join(tmp, os.path.basename(obj) + ".fatbin")
    co = os.path.join(tmp, os.path.basename(obj) + ".co")
    r = subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fb}", obj, os.devnull],
                       capture_output=True)
    if r.returncode != 0 or not os.path.exists(fb):
        return None  # no device code in this object
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o", f"--targets={TARGET}", f"--input={fb}",
                    f"--output={co}", "--unbundle"], check=True)
    return subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", co], capture_output=True,
                          text=True, check=True).stdout


def _functions(text):
    funcs, cur = {}, None
    for line in text.splitlines():
        m = _FUNC.match(line)
        if m:
            cur = funcs.setdefault(m.group(2), [])
            continue
        m = _INSN.match(line)
        if m and cur is not None:
            cur.append((int(m.group(3), 16), m.group(1), (m.group(2) or "").strip()))
    return funcs


def _hazards(insns, limit=4000):
    at = {a: i for i, (a, _, _) in enumerate(insns)}
    found = []
    for i, (addr, op, ops) in enumerate(insns):
        if op != "ds_read_b64_tr_b16":
            continue
        dest = _regs(ops.split(",")[0])
        stack, seen = [i + 1], set()
        while stack and len(seen) < limit:
            j = stack.pop()
            while j < len(insns) and j not in seen:
                seen.add(j)
                a2, op2, ops2 = insns[j]
                if op2 == "s_waitcnt" and "lgkmcnt(0)" in ops2:
                    break
                if op2 == "s_endpgm":
                    break
                if _regs(ops2) & dest:
                    found.append((hex(addr), f"{op} {ops}", hex(a2), f"{op2} {ops2}"))
                    break
                if op2.startswith("s_branch") or op2.startswith("s_cbranch"):
                    m = re.search(r"(?:<[^+>]*\+)?0x([0-9a-f]+)>?", ops2) or re.search(r"([0-9a-f]{4,})", ops2)
                    tgt = None
                    mm = re.search(r"<\S+\+0x([0-9a-f]+)>", ops2)
                    if mm:
                        tgt = insns[0][0] + int(mm.group(1), 16)
                    if tgt is not None and tgt in at:
                        stack.append(at[tgt])
                    if op2.startswith("s_branch"):
                        break
                j += 1
    return found


def test_no_inline_asm_lds_read_result_touched_before_its_wait(tmp_path):
    objs = sorted(glob.glob(os.path.join(BUILD, "kernels_*.o")))
    if not objs or not shutil.which(f"{LLVM}/llvm-objdump"):
        pytest.skip("library objects not built here (python -m dense_gemm_12_amd.build)")
    total, bad = 0, []
    for obj in objs:
        text = _disassemble(obj, str(tmp_path))
        if text is None:
            continue
        for name, insns in _functions(text).items():
            n = sum(1 for _, op, _ in insns if op == "ds_read_b64_tr_b16")
            total += n
            if n:
                h = _hazards(insns)
                if h:
                    bad.append((os.path.basename(obj), name, len(h), h[0]))
    assert total > 0, "no transposing LDS reads found: the scan is not looking at the kernels"
    assert not bad, "\n".join(f"{o} {n[:90]}: {c} hazards, first {h}" for o, n, c, h in bad[:10])
