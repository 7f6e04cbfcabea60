"""Instruction-level check of the built library's gfx950 code (CPU only).

On gfx950, with the compiler used here, a matrix instruction that reads as
its accumulator (SrcC) the result of the matrix instruction issued just
before it, when the two have different shapes (v_mfma_f32_16x16x32_bf16 and
v_mfma_f32_16x16x16_bf16, in either order), read a stale accumulator: a
one-wave probe gave wrong sums with up to 4 wait states between them and
right ones from 6, while same-shape chains were right back to back.  The
compiler inserts no wait states there.  The kernels therefore keep every
accumulation chain within one shape; this test disassembles the library's
gfx950 code objects and fails on any cross-shape accumulator dependency
closer than kMinGap wait states, so a code change cannot reintroduce one
unnoticed.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "compressed_kv_cache_amd", "libgva.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
kMinGap = 8  # wait states required (probe: 4 fail, 6 pass)

_REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)\b")


def _regs(tok):
    m = _REG.fullmatch(tok.strip())
    if not m:
        return set()
    if m.group(1):
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {(m.group(4), int(m.group(5)))}


def _dests(ins, ops):
    """Registers an instruction writes (first operand of VALU/VMEM/DS loads)."""
    if not ops:
        return set()
    if ins.startswith(("v_", "ds_read", "ds_bpermute", "ds_swizzle", "global_load",
                       "buffer_load", "flat_load", "scratch_load")):
        if ins.startswith(("v_cmp", "v_readfirstlane", "v_readlane")):
            return set()
        return _regs(ops[0])
    return set()


def cross_shape_hazards(lines, min_gap=kMinGap):
    """(function, pc, producer, consumer, gap) for every MFMA whose SrcC was
    last written by an MFMA of another opcode fewer than min_gap wait states
    before (straight-line order; s_nop n counts n + 1)."""
    out = []
    fn = None
    writer = {}  # reg -> (opcode, wait-state clock at issue)
    clock = 0
    for line in lines:
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
        if m:
            fn, writer, clock = m.group(1), {}, 0
            continue
        t = line.strip()
        if not t or t.startswith((";", "//")) or fn is None:
            continue
        body = t.split("//")[0].strip()
        if not body:
            continue
        ins = body.split()[0]
        ops = [o.strip() for o in body[len(ins):].split(",")] if len(body) > len(ins) else []
        if ins == "s_nop":
            clock += int(ops[0], 0) + 1 if ops else 1
            continue
        clock += 1
        if ins.startswith("v_mfma"):
            srcc = _regs(ops[3]) if len(ops) > 3 else set()
            for r in srcc:
                w = writer.get(r)
                if w and w[0] != ins and clock - w[1] < min_gap:
                    out.append((fn, t.split("//")[-1].strip(), w[0], ins, clock - w[1]))
                    break
            for r in _regs(ops[0]):
                writer[r] = (ins, clock)
        else:
            for r in _dests(ins, ops):
                writer.pop(r, None)
    return out


def _disassemble(tmp):
    shutil.copy(LIB, os.path.join(tmp, "libgva.so"))
    subprocess.run([OBJDUMP, "--offloading", "libgva.so"], cwd=tmp, check=True,
                   capture_output=True)
    objs = [f for f in os.listdir(tmp) if f.endswith("gfx950")]
    assert objs, "no gfx950 code object in libgva.so"
    lines = []
    for f in sorted(objs):
        r = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", f], cwd=tmp, check=True,
                           capture_output=True, text=True)
        lines += r.stdout.splitlines()
    return lines


@pytest.mark.skipif(not (os.path.exists(LIB) and os.path.exists(OBJDUMP)),
                    reason="needs the built libgva.so and llvm-objdump")
def test_no_cross_shape_accumulator_chains():
    with tempfile.TemporaryDirectory() as tmp:
        lines = _disassemble(tmp)
    n_mfma = sum(1 for l in lines if "v_mfma" in l)
    assert n_mfma > 100, "disassembly holds too few matrix instructions"
    bad = cross_shape_hazards(lines)
    assert not bad, "cross-shape MFMA accumulator chains:\n" + "\n".join(map(str, bad[:20]))


def test_scanner_flags_a_planted_chain():
    """The scanner itself: a 16x16x32 result read as SrcC by the next
    16x16x16 instruction is flagged; with 8 wait states, or through the same
    shape, it is not."""
    head = ["0000000000000000 <k>:"]
    a = "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0"
    b = "\tv_mfma_f32_16x16x16_bf16 v[12:15], v[16:17], v[18:19], v[0:3]"
    c = "\tv_mfma_f32_16x16x32_bf16 v[12:15], v[4:7], v[8:11], v[0:3]"
    assert cross_shape_hazards(head + [a, b])
    assert not cross_shape_hazards(head + [a, "\ts_nop 7", b])
    assert not cross_shape_hazards(head + [a, c])
    # a VALU write in between breaks the dependency
    assert not cross_shape_hazards(head + [a, "\tv_mov_b32_e32 v0, 0", "\tv_mov_b32_e32 v1, 0",
                                           "\tv_mov_b32_e32 v2, 0", "\tv_mov_b32_e32 v3, 0", b])
