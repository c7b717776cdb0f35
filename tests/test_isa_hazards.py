"""Static checks of the built library's gfx950 machine code (our own build,
disassembled with the ROCm LLVM tools) for two hazards of the gfx9 family
that the compiler does not cover for instructions written as inline
assembly.  Both are checked over every path that reaches an instruction
(fall-through and branches, so loop back-edges too):

1. Store data: no VALU instruction may write a data VGPR of a store wider
   than 8 bytes within the two wait states after it.  The store reads its
   data after it issues, so such a write corrupts what is stored,
   intermittently.  The compiler does not insert these wait states for buffer
   stores whose soffset is an SGPR, so the library's 16-byte epilogue stores
   carry their own.
2. SGPR operands of vector memory: a VALU instruction that writes an SGPR
   (v_readfirstlane, v_readlane -- the compiler's reload of a spilled SGPR --,
   a compare or carry-out into an SGPR pair) needs five wait states before a
   vector-memory instruction reads that SGPR as its resource, scalar offset
   or scalar address.  The compiler inserts them before the memory
   instructions it emits itself but never looks inside inline assembly.  A
   build of the dense kernel whose epilogue had a different instruction order
   put a spill reload of the row offset directly before an inline-assembly
   store in all eight transposed tensor-wise kernels, and exactly those
   kernels wrote wrong rows of D; the library's assembly blocks now start with
   enough wait states, and this check fails on any such site.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_scaled_precision_03_amd", "libmxgemm.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
STORE_WAIT_STATES = 2
SGPR_WAIT_STATES = 5

WIDE_STORE = re.compile(r"^(buffer|global|flat)_store_dwordx([34])\s+(.*)$")
VMEM = re.compile(r"^(buffer|global|scratch|flat)_\w+\s+(.*)$")
# VALU instructions whose first operand is an SGPR (or SGPR pair) they write.
VALU_SDST = re.compile(r"^(v_readlane_b32|v_readfirstlane_b32|v_cmpx?_\w+_e64|v_(add|sub|subrev)_co_u32_e64|"
                       r"v_(addc|subb|subbrev)_co_u32_e64|v_div_scale_f(32|64))\s+(.*)$")
UNCOND_END = re.compile(r"^(s_branch|s_endpgm|s_setpc_b64|s_trap)\b")
BRANCH = re.compile(r"^s_(c)?branch")


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _sregs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    if m:
        return {int(m.group(1))}
    if tok == "vcc":
        return {"vcc_lo", "vcc_hi"}
    if tok in ("vcc_lo", "vcc_hi", "m0"):
        return {tok}
    return set()


class Func:
    """One kernel: instruction texts in address order, and the predecessors
    of each instruction (the one before it unless that one ends the path,
    plus every branch that targets it)."""

    def __init__(self, name, ins):
        self.name = name
        self.text = [t for _, t, _ in ins]
        index = {a: i for i, (a, _, _) in enumerate(ins)}
        self.preds = [[] for _ in ins]
        for i, (_, t, target) in enumerate(ins):
            if i + 1 < len(ins) and not UNCOND_END.match(t):
                self.preds[i + 1].append(i)
            if target is not None and target in index:
                self.preds[index[target]].append(i)


def _parse(text):
    """llvm-objdump output -> list of Func."""
    funcs, cur, start, ins = [], None, 0, []
    for line in text.splitlines():
        m = re.match(r"^([0-9a-f]+) <(.*)>:$", line)
        if m:
            if cur is not None:
                funcs.append(Func(cur, ins))
            cur, start, ins = m.group(2), int(m.group(1), 16), []
            continue
        if cur is None or not line.startswith("\t"):
            continue
        body, _, comment = line.partition("//")
        body = body.strip()
        if not body:
            continue
        am = re.match(r"\s*([0-9A-Fa-f]+):", comment)
        addr = int(am.group(1), 16) if am else None
        target = None
        if BRANCH.match(body):
            tm = re.search(r"<[^>+]*\+0x([0-9a-f]+)>", comment)
            if tm:
                target = start + int(tm.group(1), 16)
        ins.append((addr, body, target))
    if cur is not None:
        funcs.append(Func(cur, ins))
    return funcs


def parse_listing(lines):
    """A straight-line listing (no addresses, no branches) as one Func."""
    return Func("listing", [(i, t, None) for i, t in enumerate(lines)])


def _wait_states(t):
    nop = re.match(r"s_nop\s+(0x[0-9a-f]+|\d+)", t)
    return int(nop.group(1), 0) + 1 if nop else 1


def _earlier(f, i, limit):
    """(index, wait states between it and instruction i) for every
    instruction on a path into i that lies fewer than `limit` wait states
    before it."""
    seen, out, stack = {}, [], [(p, 0) for p in f.preds[i]]
    while stack:
        j, w = stack.pop()
        if w >= limit or seen.get(j, limit + 1) <= w:
            continue
        seen[j] = w
        out.append((j, w))
        stack.extend((p, w + _wait_states(f.text[j])) for p in f.preds[j])
    return out


def _later(f, i, limit):
    """The same forward: instructions on a path out of i within `limit`."""
    succ = {}
    for j, ps in enumerate(f.preds):
        for p in ps:
            succ.setdefault(p, []).append(j)
    seen, out, stack = {}, [], [(s, 0) for s in succ.get(i, [])]
    while stack:
        j, w = stack.pop()
        if w >= limit or seen.get(j, limit + 1) <= w:
            continue
        seen[j] = w
        out.append((j, w))
        stack.extend((s, w + _wait_states(f.text[j])) for s in succ.get(j, []))
    return out


def store_hazards(f):
    """(store, writer) pairs where a VALU write hits a wide store's data
    VGPRs with fewer than STORE_WAIT_STATES wait states in between."""
    found = []
    for i, text in enumerate(f.text):
        m = WIDE_STORE.match(text)
        if not m:
            continue
        ops = [o.strip() for o in m.group(3).split(",")]
        # buffer: vdata, vaddr, ...; global/flat: vaddr, vdata, ...
        data = _vregs(ops[0] if m.group(1) == "buffer" else ops[1])
        for j, _ in _later(f, i, STORE_WAIT_STATES):
            parts = f.text[j].split(None, 1)
            if parts[0].startswith("v_") and len(parts) > 1:
                if _vregs(parts[1].split(",")[0].strip()) & data:
                    found.append((text, f.text[j]))
    return found


def sgpr_hazards(f):
    """(writer, memory instruction) pairs where a VALU write of an SGPR is
    followed by a vector-memory read of it within SGPR_WAIT_STATES."""
    found = []
    for i, text in enumerate(f.text):
        m = VMEM.match(text)
        if not m:
            continue
        reads = set()
        for o in m.group(2).split(","):
            o = o.strip().split(" ")[0] if o.strip() else ""
            reads |= _sregs(o)
        if not reads:
            continue
        for j, _ in _earlier(f, i, SGPR_WAIT_STATES):
            w = VALU_SDST.match(f.text[j])
            if w and _sregs(w.group(5).split(",")[0].strip()) & reads:
                found.append((f.text[j], text))
    return found


def _disassemble(tmp_path, lib=LIB):
    """Every gfx950 code object of the library (one offload bundle per
    translation unit, concatenated in the .hip_fatbin section), parsed."""
    fatbin = tmp_path / "fatbin.bin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section=.hip_fatbin=%s" % fatbin,
                    lib, str(tmp_path / "lib.copy")], check=True, capture_output=True)
    data = fatbin.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(b"__CLANG_OFFLOAD_BUNDLE__"), data)]
    funcs = []
    for i, st in enumerate(starts):
        part = tmp_path / ("bundle%d.bin" % i)
        part.write_bytes(data[st:starts[i + 1] if i + 1 < len(starts) else len(data)])
        code = tmp_path / ("gfx950_%d.co" % i)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--input=%s" % part, "--targets=%s" % TARGET, "--output=%s" % code],
                       check=True, capture_output=True)
        out = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", str(code)],
                             check=True, capture_output=True, text=True).stdout
        funcs += _parse(out)
    return funcs


def test_store_checker_flags_a_planted_hazard():
    planted = ["buffer_store_dwordx4 v[56:59], v238, s[12:15], s44 offen",
               "v_cndmask_b32_e64 v59, v65, v67, s[8:9]"]
    assert len(store_hazards(parse_listing(planted))) == 1
    fixed = [planted[0], "s_nop 2", planted[1]]
    assert store_hazards(parse_listing(fixed)) == []
    other = [planted[0], "v_cndmask_b32_e64 v60, v65, v67, s[8:9]", "v_mov_b32 v59, 0"]
    assert store_hazards(parse_listing(other)) == [(planted[0], "v_mov_b32 v59, 0")]


def test_sgpr_checker_flags_the_observed_hazard():
    # the site of the build whose transposed tensor-wise kernels wrote wrong rows
    seen = ["v_readlane_b32 s5, v255, 14",
            "buffer_store_dwordx4 v[48:51], v248, s[20:23], s5 offen"]
    assert len(sgpr_hazards(parse_listing(seen))) == 1
    # a reload of one SGPR of the resource, four wait states before a DMA
    dma = ["v_readfirstlane_b32 s22, v3", "s_add_u32 m0, s80, 0", "s_nop 2",
           "buffer_load_dwordx4 v6, s[20:23], 0 offen lds"]
    assert len(sgpr_hazards(parse_listing(dma))) == 1
    # five wait states clear it, as do SGPRs the memory instruction does not read
    assert sgpr_hazards(parse_listing([seen[0], "s_nop 4", seen[1]])) == []
    assert sgpr_hazards(parse_listing(["v_readlane_b32 s6, v255, 14", seen[1]])) == []
    assert sgpr_hazards(parse_listing(["s_mov_b32 s5, s7", seen[1]])) == []


def test_sgpr_checker_follows_branches():
    # a loop whose last instruction writes the SGPR that its first reads
    text = "\n".join([
        "0000000000001000 <k>:",
        "\tbuffer_load_dword v1, v2, s[8:11], s5 offen  // 000000001000: 00000000",
        "\ts_add_u32 s0, s0, 1  // 000000001008: 00000000",
        "\tv_readfirstlane_b32 s5, v3  // 00000000100C: 00000000",
        "\ts_cbranch_scc1 65531  // 000000001010: 00000000 <k+0x0>",
        "\ts_endpgm  // 000000001014: 00000000",
    ])
    (f,) = _parse(text)
    assert sgpr_hazards(f) == [("v_readfirstlane_b32 s5, v3", "buffer_load_dword v1, v2, s[8:11], s5 offen")]


needs_tools = pytest.mark.skipif(not (os.path.exists(os.path.join(LLVM, "llvm-objdump")) and os.path.exists(LIB)),
                                 reason="ROCm LLVM tools or the built library absent")


@needs_tools
def test_library_has_no_store_data_hazard(tmp_path):
    funcs = _disassemble(tmp_path)
    stores = sum(1 for f in funcs for t in f.text if WIDE_STORE.match(t))
    assert stores > 0, "no wide stores found: disassembly not parsed"
    bad = [(f.name, h) for f in funcs for h in store_hazards(f)]
    assert not bad, "%d store-data hazards, e.g. %s" % (len(bad), bad[:3])


@needs_tools
def test_library_has_no_valu_sgpr_to_vmem_hazard(tmp_path):
    funcs = _disassemble(tmp_path)
    dmas = sum(1 for f in funcs for t in f.text if VMEM.match(t) and t.endswith(" lds"))
    assert dmas > 0, "no LDS DMA found: disassembly not parsed"
    bad = [(f.name, h) for f in funcs for h in sgpr_hazards(f)]
    assert not bad, "%d VALU-SGPR -> vector-memory hazards, e.g. %s" % (len(bad), bad[:3])
    # every translation unit's kernels were seen
    names = " ".join(f.name for f in funcs)
    for k in ("dense_kernel", "dense_small_kernel", "grouped_dense_kernel", "grouped_stream_kernel",
              "quant_mx_kernel", "preshuffle_b_kernel"):
        assert k in names, k
