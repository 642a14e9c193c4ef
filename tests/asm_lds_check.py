"""Static check of the inline-assembly LDS reads in compiled kernels.

The attention kernels issue their LDS reads as inline assembly, so the
compiler does not know that a read's destination registers are filled only
when the read completes. A copy of such a register (a v_mov the register
allocator adds) before the s_waitcnt lgkmcnt that covers the read would copy
stale data. This walks a kernel's gfx950 assembly in order, models the
in-order completion of LDS operations (lgkmcnt(N) retires all but the newest
N; scalar memory loads, which share the counter, are assumed to be the
slowest so they never retire an LDS read early) and reports every
instruction that touches a register an in-flight LDS read will still write.
The walk is linear over the listing (every block as if executed in text
order), which over-approximates the pending set at a join.
"""
import re


def _regs(text):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]", text):
        for k in range(int(m.group(2)), int(m.group(3)) + 1):
            out.add(f"{m.group(1)}{k}")
    for m in re.finditer(r"\b([va])(\d+)\b", text):
        out.add(f"{m.group(1)}{m.group(2)}")
    return out


def check(asm_lines):
    """Returns a list of (line number, instruction, registers, line of the pending read)."""
    pending = []
    found = []
    for i, ln in enumerate(asm_lines):
        t = ln.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        op, args = parts[0], (parts[1] if len(parts) > 1 else "")
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", args)
            if m:
                n = int(m.group(1))
                pending = pending[len(pending) - n:] if 0 < n < len(pending) else ([] if n == 0 else pending)
            continue
        if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm"):
            continue
        used = _regs(args)
        for ln0, rs in pending:
            hit = used & rs
            if hit:
                found.append((i + 1, t, sorted(hit), ln0 + 1))
        if op.startswith("ds_read") or op.startswith("ds_load") or op.startswith("ds_bpermute") or op.startswith("ds_permute"):
            pending.append((i, _regs(args.split(",")[0])))
        elif op.startswith("ds_"):
            pending.append((i, set()))
    return found


def mfma_hazards(asm_lines, need=4):
    """VALU writes of a source register of an inline-assembly MFMA (recognised
    by its AGPR accumulator, a[...]; the compiler-built MFMAs use VGPRs and
    get their wait states from the compiler) fewer than `need` wait states
    before it. Returns (line number, MFMA, VALU instruction)."""
    found = []
    instrs = []   # (line index, op, args) of real instructions, in order
    for i, ln in enumerate(asm_lines):
        t = ln.split(";")[0].strip()
        if not t or t.startswith("."):
            continue
        if t.endswith(":"):
            instrs.append((i, ":", ""))   # label: control may join here
            continue
        parts = t.split(None, 1)
        instrs.append((i, parts[0], parts[1] if len(parts) > 1 else ""))
    for k, (i, op, args) in enumerate(instrs):
        if not (op.startswith("v_mfma") and args.split(",")[0].strip().startswith("a")):
            continue
        srcs = set()
        for operand in args.split(",")[1:3]:
            srcs |= _regs(operand)
        states = 0
        for j in range(k - 1, -1, -1):
            _, op2, args2 = instrs[j]
            if op2 == ":" or states >= need:
                break
            if op2.startswith("v_") and not op2.startswith("v_mfma"):
                if _regs(args2.split(",")[0]) & srcs:
                    found.append((i + 1, f"{op} {args}", f"{op2} {args2}"))
                    break
            states += int(args2.split()[0], 0) + 1 if op2 == "s_nop" else 1
    return found


def loads_before_first_vm_wait(asm_lines):
    """Register-destination buffer loads issued after the first inline-assembly
    LDS copy (buffer_load ... lds) and before the first s_waitcnt that counts
    vector memory operations. The compiler does not see the copies, so a
    vmcnt wait it places for one of its own loads (a spill reload, say) also
    drains every copy in flight; the kernel's query loads must all go out
    before any such wait for their latency to overlap that of the first KV
    tiles. Returns (number of such loads, line number of the wait or None)."""
    started, n = False, 0
    for i, ln in enumerate(asm_lines):
        t = ln.split(";")[0].strip()
        if not t.startswith(("buffer_load", "s_waitcnt")):
            continue
        if t.startswith("buffer_load"):
            if t.endswith(" lds"):
                started = True
            elif started:
                n += 1
        elif started and "vmcnt" in t:
            return n, i + 1
    return n, None


def kernel_lines(asm_text, symbol_prefix):
    """Lines of the first function whose symbol starts with symbol_prefix."""
    out, inside = [], False
    for ln in asm_text.split("\n"):
        if not inside and ln.startswith(symbol_prefix) and ln.split(";")[0].rstrip().endswith(":"):
            inside = True
        if inside:
            out.append(ln)
            if "s_endpgm" in ln:
                break
    return out
