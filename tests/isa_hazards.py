"""Static check of matrix-product result reads in gfx950 device assembly.

A matrix-core product (v_mfma_*) writes its result registers some cycles
after it issues, and the hardware does not stall a vector instruction that
reads them early: the program must leave enough wait states (instructions,
or s_nop N = N + 1 states) in between.  The compiler counts them, but its
count has been seen to fall short on a loop-exit path.  This module walks the
control-flow graph of each kernel and reports every read of a product's
result register (by a vector, memory or AGPR-copy instruction, or as the A/B
operand of another product) whose distance from the product, minimised over
all paths, is below the requirement.  Chained accumulation (the register as
the C operand of the next product) is interlocked and not checked.

Requirements used: the wait states the compiler itself puts between a
product and a read of its result in straight-line gfx950 code (s_nop 15 +
s_nop 1 = 18 for the fp32 32x32x2 product, s_nop 11 = 12 for the bf16
32x32x16 product, s_nop 9 = 10 for the fp32 16x16x4 product, s_nop 7 = 8
for the bf16 16x16x32 product), the same for
a vector, store, LDS-write, AGPR-copy or product-operand read.

The reverse direction is checked too: a product that reads an operand (A, B
or the accumulator C) written by a vector instruction needs 2 wait states
after it (the compiler emits s_nop 0 plus the s_waitcnt before the product,
or s_nop 1).  The compiler counts both for its own products; products
written as inline assembly are counted by nobody but this check.
"""
from __future__ import annotations

import re
from collections import defaultdict

NEED = {
    "v_mfma_f32_32x32x2_f32": 18,
    "v_mfma_f32_32x32x16_bf16": 12,
    "v_mfma_f32_16x16x4_f32": 10,
    "v_mfma_f32_16x16x32_bf16": 8,
}
DEFAULT_NEED = 18  # unknown products: the longest requirement above
VALU_TO_PRODUCT = 2


def need_of(op: str) -> int:
    return NEED.get(op, DEFAULT_NEED)


def registers(tok: str) -> list[tuple[str, int]]:
    m = re.fullmatch(r"([va])(\d+)", tok)
    if m:
        return [(m.group(1), int(m.group(2)))]
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return [(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)]
    return []


def split_functions(text: str) -> dict[str, list[tuple[str, str]]]:
    """{kernel symbol: [("label", name) | ("ins", text)]} for every function."""
    funcs: dict[str, list] = {}
    cur = None
    for raw in text.splitlines():
        code = raw.split(";")[0].rstrip()
        if re.match(r"^_Z\S*:$", code):
            cur = funcs.setdefault(code[:-1], [])
            continue
        if cur is None:
            continue
        if code.startswith(".Lfunc_end"):
            cur = None
            continue
        if re.match(r"^\.LBB\S*:$", code):
            cur.append(("label", code[:-1]))
            continue
        if raw.strip().startswith("; %bb."):
            cur.append(("label", raw.strip()))
            continue
        code = code.strip()
        if code and not code.startswith("."):
            cur.append(("ins", code))
    return funcs


def _ops(ins: str) -> tuple[str, list[str]]:
    parts = ins.replace(",", " ").split()
    return parts[0], parts[1:]


def _is_store(op: str) -> bool:
    return op.startswith(("ds_write", "global_store", "buffer_store", "flat_store", "scratch_store"))


def check_function(items: list[tuple[str, str]]) -> list[tuple[str, str, tuple[str, int], int, int]]:
    """Violations (block label, instruction, register, wait states, needed)."""
    blocks: list[dict] = []
    blk = {"label": None, "ins": []}
    for kind, x in items:
        if kind == "label":
            if blk["ins"] or blk["label"]:
                blocks.append(blk)
            blk = {"label": x, "ins": []}
            continue
        blk["ins"].append(x)
        op = x.split()[0]
        if op.startswith(("s_branch", "s_cbranch", "s_setpc")) or op == "s_endpgm":
            blocks.append(blk)
            blk = {"label": None, "ins": []}
    if blk["ins"] or blk["label"]:
        blocks.append(blk)
    index = {b["label"]: i for i, b in enumerate(blocks) if b["label"]}
    preds: dict[int, list[int]] = defaultdict(list)
    for i, b in enumerate(blocks):
        last = b["ins"][-1].split() if b["ins"] else ["s_nop"]
        op = last[0]
        if op == "s_branch":
            preds[index[last[1]]].append(i)
        elif op.startswith("s_cbranch"):
            preds[index[last[1]]].append(i)
            preds[i + 1].append(i)
        elif op == "s_endpgm" or op.startswith("s_setpc"):
            pass
        else:
            preds[i + 1].append(i)

    def states(ins: str) -> int:
        op, ops = _ops(ins)
        return int(ops[0], 0) + 1 if op == "s_nop" else 1

    def writer_need(op: str, valu: bool):
        """Wait states a reader needs after a write by op: products (valu
        False) or vector instructions (valu True); None for other writers."""
        if op.startswith("v_mfma"):
            return None if valu else need_of(op)
        if valu and op.startswith("v_"):
            return VALU_TO_PRODUCT
        return None

    def nearest(bi: int, pos: int, reg, budget: int, seen: frozenset, valu: bool = False):
        """(wait states, needed) of the closest writer of reg before (bi, pos)
        on any path that is a product (valu False) or a vector instruction
        (valu True), minimising wait states - needed; None if there is none
        within budget or another instruction writes reg first."""
        dist = 0
        lst = blocks[bi]["ins"]
        for j in range(pos - 1, -1, -1):
            op, ops = _ops(lst[j])
            if ops and not op.startswith("s_") and not _is_store(op) and reg in registers(ops[0]):
                need = writer_need(op, valu)
                return None if need is None else (dist, need)
            dist += states(lst[j])
            if dist >= budget:
                return None
        best = None
        for p in preds.get(bi, []):
            if (p, reg) in seen:
                continue
            r = nearest(p, len(blocks[p]["ins"]), reg, budget - dist, seen | {(p, reg)}, valu)
            if r is not None:
                r = (r[0] + dist, r[1])
                if best is None or r[0] - r[1] < best[0] - best[1]:
                    best = r
        return best

    budget = max(NEED.values()) + 1
    out = []
    for bi, b in enumerate(blocks):
        for j, ins in enumerate(b["ins"]):
            op, ops = _ops(ins)
            if op.startswith("s_") or not ops:
                continue
            if op.startswith("v_mfma"):
                srcs = ops[1:3]
            elif _is_store(op):
                srcs = ops
            else:
                srcs = ops[1:]
            for tok in srcs:
                for reg in registers(tok):
                    r = nearest(bi, j, reg, budget, frozenset())
                    if r is not None and r[0] < r[1]:
                        out.append((b["label"], ins, reg, r[0], r[1]))
            if op.startswith("v_mfma"):
                for tok in ops[1:4]:
                    for reg in registers(tok):
                        r = nearest(bi, j, reg, VALU_TO_PRODUCT + 1, frozenset(), valu=True)
                        if r is not None and r[0] < r[1]:
                            out.append((b["label"], ins, reg, r[0], r[1]))
    return out


def check_text(text: str) -> dict[str, list]:
    """{kernel: violations} for every function with at least one."""
    res = {}
    for name, items in split_functions(text).items():
        v = check_function(items)
        if v:
            res[name] = v
    return res
