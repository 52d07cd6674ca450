"""Wait-state check of the direct-to-LDS loads in the built gfx950 code.

The forward issues its K/V loads (`buffer_load_dwordx4 ... lds`) from inline
asm, which the compiler's hazard recognizer does not look into.  The asm
block therefore brings its own wait states, and this module checks on the
disassembled library that they suffice on every path into every such load.
The rules, from the CDNA3/CDNA4 ISA "manually inserted wait states" table,
the same ones the compiler applies to its own LDS-DMA loads:

- M0 written by a scalar instruction, then read by an LDS-DMA load: 1 wait state;
- an SGPR written by a vector instruction (v_readlane, v_readfirstlane,
  v_cmp, a carry-out ...), then read by a vector-memory instruction: 5 wait
  states (this covers M0 too);
- a VGPR written by a matrix instruction, then read as a vector-memory
  address: up to 19 wait states on this family; the address registers are
  held constant, so the check asks for that much.

Each issued instruction counts one wait state; `s_nop N` counts N + 1.  The
distances are propagated over the control-flow graph (branch targets and
fall-through), taking the minimum over all predecessors of a block.
"""

import os
import re
import struct
import subprocess

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NEED_VALU_SGPR = 5
NEED_M0 = 1
NEED_VGPR = 19
_CAP = max(NEED_VALU_SGPR, NEED_M0, NEED_VGPR)


def code_objects(so_path, tmp_dir, arch="gfx950"):
    """The device code objects (ELF bytes) for `arch` in a HIP shared library."""
    fat_path = os.path.join(tmp_dir, "fatbin")
    subprocess.run([LLVM + "/llvm-objcopy", "--dump-section", ".hip_fatbin=" + fat_path, so_path,
                    os.path.join(tmp_dir, "stripped.so")], check=True)
    with open(fat_path, "rb") as f:
        fat = f.read()
    out = []
    for s in range(0, len(fat), 8):
        if fat[s:s + len(MAGIC)] != MAGIC:
            continue
        n, = struct.unpack_from("<Q", fat, s + 24)
        p = s + 32
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", fat, p)
            p += 24
            triple = fat[p:p + tl].decode()
            p += tl
            if triple.endswith("--" + arch) and size:
                out.append(fat[s + off:s + off + size])
    return out


def disassemble(elf, path, arch="gfx950"):
    with open(path, "wb") as f:
        f.write(elf)
    return subprocess.run([LLVM + "/llvm-objdump", "-d", "--mcpu=" + arch, path], stdout=subprocess.PIPE,
                          check=True, text=True).stdout


_FUNC = re.compile(r"^([0-9a-f]+) <(.+)>:$")
_INST = re.compile(r"^\s+(\S+)(.*?)\s*//\s*([0-9A-Fa-f]+):")
_TARGET = re.compile(r"<(.+)\+0x([0-9a-f]+)>")


def functions(text):
    """{name: [(addr, mnemonic, operand string, branch target addr or None)]}."""
    funcs, cur, base = {}, None, 0
    for line in text.split("\n"):
        m = _FUNC.match(line)
        if m:
            base, cur = int(m.group(1), 16), m.group(2)
            funcs[cur] = []
            continue
        m = _INST.match(line)
        if m and cur is not None:
            ops = m.group(2).strip()
            tgt = None
            if m.group(1).startswith(("s_branch", "s_cbranch")):
                t = _TARGET.search(line)
                tgt = base + int(t.group(2), 16) if t and t.group(1) == cur else -1
            funcs[cur].append((int(m.group(3), 16), m.group(1), ops, tgt))
    return funcs


def _regs(tok):
    """Register names in one operand: s5 / s[4:7] / v3 / v[2:5] / m0 / vcc."""
    tok = tok.strip()
    m = re.fullmatch(r"([sva])(\d+)", tok)
    if m:
        return [tok]
    m = re.fullmatch(r"([sva])\[(\d+):(\d+)\]", tok)
    if m:
        return ["%s%d" % (m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)]
    if tok in ("m0", "exec", "exec_lo", "exec_hi", "vcc", "vcc_lo", "vcc_hi"):
        return [tok]
    return []


def _split_ops(ops):
    out, depth, cur = [], 0, ""
    for c in ops:
        if c == "[":
            depth += 1
        elif c == "]":
            depth -= 1
        if c == "," and depth == 0:
            out.append(cur)
            cur = ""
        else:
            cur += c
    if cur.strip():
        out.append(cur)
    return [o.strip().split(" ")[0] for o in out]


# scalar instructions whose first operand is not a register they write
_S_NO_DEF = ("s_branch", "s_cbranch", "s_waitcnt", "s_nop", "s_barrier", "s_setprio", "s_sendmsg", "s_endpgm",
             "s_dcache", "s_icache", "s_sleep", "s_cmp", "s_bitcmp", "s_setreg", "s_set_gpr_idx", "s_store",
             "s_buffer_store", "s_scratch_store", "s_atc", "s_ttrace", "s_setvskip", "s_trap", "s_incperflevel",
             "s_decperflevel", "s_setkill", "s_setpc", "s_rfe")
_VOP3B = re.compile(r"v_(add|sub|subrev)_co_|v_(addc|subb|subbrev)_co_|v_div_scale|v_mad_(u64_u32|i64_i32)")


def _defs(mn, ops):
    """(registers a vector instruction writes, registers written otherwise)."""
    o = _split_ops(ops)
    if not o:
        return [], []
    d0 = _regs(o[0])
    if mn.startswith("v_"):
        d = list(d0)
        if _VOP3B.match(mn) and len(o) > 1:
            d += [r for r in _regs(o[1]) if not r.startswith("v")]
        if mn.startswith("v_cmpx"):
            d.append("exec")
        return d, []
    if mn.startswith(("s_movreld", "s_movrels")):
        raise ValueError("indexed SGPR move: not analysed")
    if mn.startswith("s_") and not mn.startswith(_S_NO_DEF):
        return [], d0
    if mn.startswith(("buffer_load", "global_load", "flat_load", "ds_read", "ds_bpermute", "ds_permute",
                      "scratch_load")) and " lds" not in " " + ops:
        return [], d0
    return [], []


def _waits(mn, ops):
    if mn == "s_nop":
        return int(ops.split()[0], 0) + 1
    return 1


def is_lds_dma(mn, ops):
    return mn.startswith(("buffer_load", "global_load")) and re.search(r"\blds\b", ops) is not None


def check_function(insts):
    """Violations [(addr, text)] of the LDS-DMA wait-state rules in one function."""
    if not insts:
        return []
    # registers read by the LDS-DMA loads: the only ones tracked
    tracked = set(["m0"])
    for _, mn, ops, _ in insts:
        if is_lds_dma(mn, ops):
            o = _split_ops(ops)
            tracked.update(_regs(o[0]))
            tracked.update(_regs(o[1]))
            if len(o) > 2:
                tracked.update(_regs(o[2]))
    addr_idx = {a: i for i, (a, _, _, _) in enumerate(insts)}
    leaders = {0}
    for i, (_, mn, _, tgt) in enumerate(insts):
        if tgt is not None:
            if tgt not in addr_idx:
                return [(insts[i][0], "branch to an unknown target: %s" % mn)]
            leaders.add(addr_idx[tgt])
            leaders.add(i + 1)
        if mn in ("s_endpgm", "s_setpc_b64", "s_swappc_b64"):
            leaders.add(i + 1)
    starts = sorted(x for x in leaders if x < len(insts))
    blocks = [(s, (starts[k + 1] if k + 1 < len(starts) else len(insts))) for k, s in enumerate(starts)]
    bidx = {s: k for k, (s, _) in enumerate(blocks)}
    succ = []
    for s, e in blocks:
        _, mn, _, tgt = insts[e - 1]
        out = []
        if tgt is not None:
            out.append(bidx[addr_idx[tgt]])
        if mn in ("s_setpc_b64", "s_swappc_b64"):
            return [(insts[e - 1][0], "indirect branch: not analysed")]
        if not (mn == "s_branch" or mn == "s_endpgm") and e < len(insts):
            out.append(bidx[e])
        succ.append(out)
    # state: {("valu"|"any", reg): wait states since that kind of write}; absent = far
    def transfer(k, state, report):
        st = dict(state)
        s, e = blocks[k]
        for i in range(s, e):
            a, mn, ops, _ = insts[i]
            if report is not None and is_lds_dma(mn, ops):
                o = _split_ops(ops)
                for r in _regs(o[1]) + (_regs(o[2]) if len(o) > 2 else []) + ["m0"]:
                    if st.get(("valu", r), _CAP) < NEED_VALU_SGPR:
                        report.append((a, "%s: %s written by a vector instruction %d wait states before"
                                       % (mn, r, st[("valu", r)])))
                if st.get(("any", "m0"), _CAP) < NEED_M0:
                    report.append((a, "%s: m0 written %d wait states before" % (mn, st[("any", "m0")])))
                for r in _regs(o[0]):
                    if st.get(("any", r), _CAP) < NEED_VGPR:
                        report.append((a, "%s: address %s written %d wait states before"
                                       % (mn, r, st[("any", r)])))
            w = _waits(mn, ops)
            for key in list(st):
                st[key] = min(_CAP, st[key] + w)
            vdefs, odefs = _defs(mn, ops)
            for r in vdefs:
                if r in tracked:
                    st[("valu", r)] = 0
                    st[("any", r)] = 0
            for r in odefs:
                if r in tracked:
                    st[("any", r)] = 0
                    st.pop(("valu", r), None)   # the last writer is not a vector instruction
            for key in [k2 for k2, v in st.items() if v >= _CAP]:
                del st[key]
        return st

    inn = [None] * len(blocks)
    inn[0] = {}
    work = [0]
    while work:
        k = work.pop()
        out = transfer(k, inn[k], None)
        for j in succ[k]:
            if inn[j] is None:
                new = dict(out)
            else:
                new = dict(inn[j])
                for key in set(new) | set(out):
                    new[key] = min(new.get(key, _CAP), out.get(key, _CAP))
                new = {key: v for key, v in new.items() if v < _CAP}
            if new != inn[j]:
                inn[j] = new
                work.append(j)
    report = []
    for k in range(len(blocks)):
        if inn[k] is not None:
            transfer(k, inn[k], report)
    return report


def check_library(so_path, tmp_path):
    """{function: (number of LDS-DMA loads, violations)} over every device function."""
    res = {}
    for n, elf in enumerate(code_objects(so_path, tmp_path)):
        text = disassemble(elf, "%s/co%d.o" % (tmp_path, n))
        for name, insts in functions(text).items():
            nd = sum(1 for _, mn, ops, _ in insts if is_lds_dma(mn, ops))
            if nd:
                res[name] = (nd, check_function(insts))
    return res
