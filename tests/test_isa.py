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


# ---- the split-merge protocol and register spills of the decode kernels ----
#
# Each block of the split decode stores its partial record, every thread
# waits until its stores are acknowledged (s_waitcnt vmcnt(0): on gfx9 the
# counter also covers stores), the block meets at a barrier, and one thread
# takes a ticket with an atomic add; the block drawing the last ticket loads
# every record of its sequence.  The records are written and read with the
# device-scope coherence bit (sc1: stores go through the XCD's L2 to memory,
# loads do not take a line the local L2 may hold), and the atomic is
# performed at the memory side of every XCD's L2.  So the atomic of each
# block follows the acknowledgement of that block's records, and the last
# block's loads read what those stores wrote, whichever XCDs ran the
# blocks.  These checks pin that instruction sequence in the built library.

def _functions(lines):
    """{function name: [(address, instruction text, branch target or None)]}
    from llvm-objdump's listing (addresses and targets from its comments)."""
    out, fn, base = {}, None, 0
    for line in lines:
        m = re.match(r"^([0-9a-f]+) <(.+)>:$", line)
        if m:
            base, fn = int(m.group(1), 16), m.group(2)
            out[fn] = []
            continue
        if fn is None or not line.strip():
            continue
        text, _, comment = line.strip().partition("//")
        text = text.strip()
        ma = re.match(r"\s*([0-9A-Fa-f]+):", comment)
        if not text or not ma:
            continue
        mt = re.search(r"<[^>+]+\+0x([0-9a-f]+)>", comment)
        target = base + int(mt.group(1), 16) if mt and text.startswith("s_") and \
            "branch" in text.split()[0] else None
        out[fn].append((int(ma.group(1), 16), text, target))
    return out


def _is_store(t):
    return re.match(r"(global|buffer|flat)_store", t) is not None


def _falls_through(t):
    return not t.startswith(("s_branch", "s_endpgm", "s_setpc"))


def merge_protocol_violations(body):
    """Violations in one decode kernel, following control flow: on every
    path into a ticket atomic (global_atomic_add), the nearest device-scope
    (sc1) store -- a record -- must be followed by s_waitcnt vmcnt(0) and
    then s_barrier before the atomic; some path must reach one; and every
    load reachable from a ticket must carry sc1.  Plain stores (the outputs
    of an empty sequence, under an exec mask that leaves the ticket idle)
    are passed over."""
    text = [t for _, t, _ in body]
    at = {addr: i for i, (addr, _, _) in enumerate(body)}
    preds = {i: [] for i in range(len(body))}
    succs = {i: [] for i in range(len(body))}
    for i, (_, t, tgt) in enumerate(body):
        if i + 1 < len(body) and _falls_through(t):
            preds[i + 1].append(i)
            succs[i].append(i + 1)
        if tgt is not None and tgt in at:
            preds[at[tgt]].append(i)
            succs[i].append(at[tgt])
    tickets = [i for i, t in enumerate(text) if t.startswith("global_atomic_add")]
    if not tickets:
        return ["no ticket atomic"]
    bad = []
    for i in tickets:
        stack, seen, met = [(p, False, False) for p in preds[i]], set(), 0
        while stack:
            j, barrier, wait = stack.pop()
            if (j, barrier, wait) in seen:
                continue
            seen.add((j, barrier, wait))
            t = text[j]
            if _is_store(t) and " sc1" in t:
                met += 1
                if not (barrier and wait):
                    bad.append(f"record store on a path into the ticket at {i} not fenced: {t}")
                continue
            if t.startswith("s_barrier"):
                barrier = True
            elif barrier and t.startswith("s_waitcnt") and "vmcnt(0)" in t:
                wait = True
            stack += [(p, barrier, wait) for p in preds[j]]
        if not met:
            bad.append(f"no device-scope record store reaches the ticket at {i}")
    reach, stack = set(), list(tickets)
    while stack:
        j = stack.pop()
        if j in reach:
            continue
        reach.add(j)
        stack += succs[j]
    for j in sorted(reach):
        if re.match(r"(global|buffer|flat)_load", text[j]) and " sc1" not in text[j]:
            bad.append(f"record load without sc1: {text[j]}")
    return bad


def spill_sites(body):
    return [t for _, t, _ in body if t.startswith("scratch_")]


# The GQA context kernel at d_h = 128 keeps two register sets of key and
# value tiles (256 registers of tile data); it spills 44 bytes per lane.  It
# is the same-shape comparison kernel, not a step of the method, and reads
# the larger-model shape's cache at 98 % of a plain read of 1 GiB despite
# the spill.
KNOWN_SPILLS = ("decode_mfma_kernel<4, 128, 0, true, 4, 1, 2,",)


def _demangled(name):
    r = subprocess.run(["c++filt", name], capture_output=True, text=True)
    d = r.stdout.strip().replace("gva::(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", d).replace("void ", "")


@pytest.mark.skipif(not (os.path.exists(LIB) and os.path.exists(OBJDUMP)),
                    reason="needs the built libgva.so and llvm-objdump")
def test_decode_merge_protocol_and_no_spills():
    with tempfile.TemporaryDirectory() as tmp:
        fns = _functions(_disassemble(tmp))
    decode = {n: b for n, b in fns.items() if "decode_mfma_kernel" in n}
    assert len(decode) >= 30, "fewer decode kernel instances than expected"
    problems = []
    for name, body in decode.items():
        pretty = _demangled(name)
        problems += [f"{pretty}: {p}" for p in merge_protocol_violations(body)]
        if spill_sites(body) and not pretty.startswith(KNOWN_SPILLS):
            problems.append(f"{pretty}: spills to scratch")
    assert not problems, "\n".join(problems[:20])


def test_protocol_checker_flags_planted_mistakes():
    def fn(*ins):
        return [(4 * k, t, None) for k, t in enumerate(ins)]
    st = "global_store_dwordx2 v0, v[2:3], s[0:1] sc1"
    tk = "global_atomic_add v1, v1, v2, s[4:5] sc0"
    ld = "global_load_dwordx2 v[4:5], v0, s[6:7] sc1"
    assert not merge_protocol_violations(fn(st, "s_waitcnt vmcnt(0)", "s_barrier", tk, ld))
    assert merge_protocol_violations(fn(st, "s_barrier", tk, ld))             # no wait
    assert merge_protocol_violations(fn(st, "s_barrier", "s_waitcnt vmcnt(0)", tk, ld))
    assert merge_protocol_violations(fn(st.replace(" sc1", ""), "s_waitcnt vmcnt(0)",
                                        "s_barrier", tk, ld))                # plain record
    assert merge_protocol_violations(fn(st, "s_waitcnt vmcnt(0)", "s_barrier", tk,
                                        ld.replace(" sc1", "")))             # plain load
    # a branch around the fence into the ticket is followed
    body = [(0, st, None), (4, "s_cbranch_scc0 2", 16), (8, "s_waitcnt vmcnt(0)", None),
            (12, "s_barrier", None), (16, tk, None)]
    assert merge_protocol_violations(body)
    assert spill_sites(fn("scratch_store_dword off, v3, s33"))
