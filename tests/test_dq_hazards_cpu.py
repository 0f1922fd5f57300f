"""Wait states around the dQ kernel's inline-assembly matrix products,
checked on the gfx950 assembly of the kernel as built (no GPU needed).

The dQ kernel (csrc/bwd.hip) writes its products as inline assembly so that
long-lived operands and accumulators stay in AGPRs.  The compiler places no
wait states around instructions it cannot see into, so the kernel places
them itself (mfma_settle, mfma_settle_short, agpr_settle in csrc/stage.h).
This test compiles bwd.hip with the library's flags to assembly and walks
the control-flow graph from every inline product, in both directions:

  * after the product: every path must issue at least RAW_MIN wait states
    (one per instruction, N + 1 per s_nop N) before a non-product vector or
    memory instruction reads or writes any register of its result;
  * before the product: every path back must hold at least VALU_MIN wait
    states between the last vector write of one of its operands (A, B or the
    accumulator) and the product.

The limits follow the matrix-core dependency rules the compiler applies
for gfx950 to the products it can see: an 8-pass 32x32x16 product's result
may be touched by vector code (v_accvgpr_read included) after passes + 4 =
12 wait states; a vector write of an operand needs 2 before the product,
here rounded up to 4.  Every intervening instruction counts one wait state
and an intervening product its 8 passes: the matrix pipe takes a 32x32x16
product only every 8 passes (its peak rate), so a product issued between
the producer and the reader delays the reader at least that long.  Operands
loaded from memory are covered by the waitcnt the compiler places for the
asm's inputs, so loads are not counted as writes here.  The closest cases
in the kernel as built are the copies of the dQ accumulators out of the
AGPRs after the walk, which the register allocator places right after the
last products (behind the products into the other accumulators)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RAW_MIN = 12
VALU_MIN = 4
PRODUCT_PASSES = 8  # a 32x32x16 fp16 product on gfx950
HORIZON = 96  # wait states after which no hazard remains


def _regs(tok):
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _parse(text):
    """Instructions of each kernel: (op, args, inline, label) in order."""
    kernels, cur, inline = {}, None, False
    for ln in text.split("\n"):
        s = ln.strip()
        m = re.match(r"^(_Z\S*dq_kernel\S*):", s)
        if m:
            cur = kernels.setdefault(m.group(1), [])
            continue
        if cur is None:
            continue
        if s.startswith(";;#ASMSTART"):
            inline = True
            continue
        if s.startswith(";;#ASMEND"):
            inline = False
            continue
        m = re.match(r"^(\.LBB\S+):", s)
        if m:
            cur.append(("label", [m.group(1)], False))
            continue
        if not s or s.startswith((";", ".")):
            continue
        s = s.split(";")[0].strip()
        op = s.split()[0]
        args = [a.strip() for a in s[len(op):].split(",")] if len(s) > len(op) else []
        cur.append((op, args, inline))
        if op == "s_endpgm":
            cur = None
    return kernels


def _defs_uses(op, args):
    regs = [_regs(a) for a in args]
    if op.startswith(("ds_write", "global_store", "buffer_store", "flat_store")):
        return set(), set().union(*regs) if regs else set()
    if op.startswith(("v_", "ds_", "global_", "buffer_", "flat_")) and regs:
        return regs[0], set().union(*regs[1:]) if len(regs) > 1 else set()
    return set(), set()


def _waits(op, args):
    if op == "s_nop":
        return int(args[0], 0) + 1
    if op.startswith("v_mfma_f32_32x32x16"):
        return PRODUCT_PASSES  # the matrix pipe takes the next product after these passes
    return 0 if op == "label" else 1


def _succ(ins, labels, i):
    op, args, _ = ins[i]
    if op in ("s_endpgm", "s_setpc_b64"):
        return []
    if op == "s_branch":
        return [labels[args[0]]]
    if op.startswith("s_cbranch"):
        return [labels[args[0]], i + 1]
    return [i + 1] if i + 1 < len(ins) else []


def _check(ins):
    labels = {a[0]: i for i, (op, a, _) in enumerate(ins) if op == "label"}
    preds = {i: [] for i in range(len(ins))}
    for i in range(len(ins)):
        for j in _succ(ins, labels, i):
            preds[j].append(i)
    min_after, min_before, products = 10 ** 9, 10 ** 9, 0
    for i, (op, args, inline) in enumerate(ins):
        if not (inline and op.startswith("v_mfma")):
            continue
        products += 1
        D = _regs(args[0])
        src = set().union(*[_regs(a) for a in args[1:4]])
        # forward: first access to the result on every path
        stack, seen = [(j, 0) for j in _succ(ins, labels, i)], set()
        while stack:
            j, ws = stack.pop()
            if (j, ws) in seen or ws >= HORIZON:
                continue
            seen.add((j, ws))
            op2, a2, _ = ins[j]
            d2, u2 = _defs_uses(op2, a2)
            if not op2.startswith("v_mfma") and (d2 | u2) & D:
                min_after = min(min_after, ws)
                continue
            stack += [(k, ws + _waits(op2, a2)) for k in _succ(ins, labels, j)]
        # backward: last vector write of an operand on every path
        stack, seen = [(j, 0) for j in preds[i]], set()
        while stack:
            j, ws = stack.pop()
            if (j, ws) in seen or ws >= HORIZON:
                continue
            seen.add((j, ws))
            op2, a2, _ = ins[j]
            d2, _ = _defs_uses(op2, a2)
            if op2.startswith("v_") and not op2.startswith("v_mfma") and d2 & src:
                min_before = min(min_before, ws)
                continue
            stack += [(k, ws + _waits(op2, a2)) for k in preds[j]]
    return products, min_after, min_before


@pytest.fixture(scope="module")
def dq_asm(tmp_path_factory):
    from block_diffusion_lm_bdlm_amd import build as lb
    out = str(tmp_path_factory.mktemp("asm") / "bwd.s")
    cmd = [lb._hipcc(), "-x", "hip", "-S", "--cuda-device-only", os.path.join(lb.CSRC, "bwd.hip"), "-o", out] \
        + lb._flags() + lb.EXTRA["bwd.hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-2000:])
    return open(out).read()


def test_inline_products_keep_their_wait_states(dq_asm):
    kernels = _parse(dq_asm)
    assert len(kernels) == 2, list(kernels)  # d = 64 and d = 128
    for name, ins in kernels.items():
        products, after, before = _check(ins)
        print(f"{name}: {products} inline products; min wait states product -> vector access {after}, "
              f"vector write -> product {before}")
        assert products >= 96
        assert after >= RAW_MIN, (name, after)
        assert before >= VALU_MIN, (name, before)
