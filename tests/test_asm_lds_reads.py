"""Inline-asm LDS reads must not share registers with other work while in flight.

The 256x256 expert GEMM and the fused router read their MFMA operands from
LDS with inline `ds_read_b128` statements, so the compiler cannot put its own
waits between them and the multiplies. The compiler takes an asm output as
written when the statement issues; if nothing uses that output it treats the
registers as free and may give them to other values while the read is still in
flight, and the read then lands on top of them (an address, a row index: a
memory fault on the GPU). The code guards against this by consuming every read
in a multiply and by tying each wait to the registers it covers.

This test compiles both sources for gfx950 to assembly (no GPU needed) and
replays every function's instruction stream in text order with an in-order
model of the LDS queue: each `ds_*` instruction joins the queue, and
`s_waitcnt lgkmcnt(N)` leaves at most the N youngest in flight (LDS operations
complete in order; scalar loads also count against lgkmcnt, which only makes
the N youngest a safe over-estimate). Any instruction that reads or writes a
register of an inline-asm read still in flight is a hazard; back-to-back
inline reads into the same registers are not (they land in order). Branches
are ignored: text order is one path through each function, and the kernels'
hot loops run in that order. A copy of the GEMM whose down-projection epilogue
does nothing (so its multiplies are dead code and the operand reads lose their
only users) must be flagged: the check sees the mistake it is for.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from top_routed_expert_amd import build as B

REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def regs_of(text: str) -> set:
    out = set()
    for a, b, c in REG.findall(text):
        if c:
            out.add(int(c))
        else:
            out |= set(range(int(a), int(b) + 1))
    return out


def lds_hazards(asm: str) -> dict:
    """{function: [(line of the read, line of the clash, instruction)]} over an assembly listing."""
    res, cur, queue, in_asm = {}, None, [], False
    for i, raw in enumerate(asm.splitlines()):
        s = raw.strip()
        m = re.match(r"^(_Z\S+):", raw)
        if m:
            cur, queue = m.group(1), []
            res[cur] = []
            continue
        if cur is None:
            continue
        if s == ";;#ASMSTART":
            in_asm = True
            continue
        if s == ";;#ASMEND":
            in_asm = False
            continue
        if raw.startswith(".Lfunc_end"):
            cur = None
            continue
        ins = s.split(";")[0].strip()
        if not ins or ins.endswith(":") or ins.startswith("."):
            continue
        op = ins.split()[0]
        if op == "s_endpgm":
            queue = []
            continue
        if op.startswith("s_waitcnt"):
            w = re.search(r"lgkmcnt\((\d+)\)", ins)
            if w:
                n = int(w.group(1))
                queue = queue[len(queue) - n:] if 0 < n < len(queue) else ([] if n == 0 else queue)
            continue
        used = regs_of(ins)
        inline_read = op.startswith("ds_read") and in_asm
        for regs, at in queue:
            if regs and used & regs and not inline_read:
                res[cur].append((at, i, ins))
        if op.startswith("ds_"):
            dst = set()
            if inline_read:
                d = re.match(r"ds_read\S*\s+(v\[\d+:\d+\]|v\d+)", ins)
                dst = regs_of(d.group(1))
            queue.append((dst, i))
    return res


def device_asm(src_path: str, out_path: str) -> str:
    cmd = [B.hipcc(), *B.FLAGS, "--cuda-device-only", "-S", src_path, "-o", out_path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out_path).read()


DEAD_EPILOGUE = ("""    } else {
      // 16 rows x 64 fp32 columns; 16-column groups XOR-swizzled by (row >> 2) & 3
""", """    } else {
      return;
      // 16 rows x 64 fp32 columns; 16-column groups XOR-swizzled by (row >> 2) & 3
""")


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    big8 = os.path.join(B.CSRC, "grouped_gemm_big8.hip")
    src = open(big8).read()
    assert DEAD_EPILOGUE[0] in src, "the down-projection epilogue moved: update the planted copy"
    planted = d / "big8_dead_epilogue.hip"
    planted.write_text(src.replace(*DEAD_EPILOGUE))
    jobs = {"big8": big8, "router": os.path.join(B.CSRC, "router.hip"), "planted": str(planted)}
    with cf.ThreadPoolExecutor(3) as ex:
        futs = {k: ex.submit(device_asm, v, str(d / f"{k}.s")) for k, v in jobs.items()}
        return {k: f.result() for k, f in futs.items()}


@pytest.mark.parametrize("name", ["big8", "router"])
def test_inline_lds_reads_keep_their_registers(listings, name):
    res = lds_hazards(listings[name])
    kernels = [f for f in res if "gemm_bf16_big8" in f or "router_topk" in f]
    assert kernels, f"no kernels found in {name}"
    bad = {f: v for f, v in res.items() if v}
    assert not bad, "registers of in-flight LDS reads reused: " + "; ".join(
        f"{f}: read at line {v[0][0]} clashes with `{v[0][2]}`" for f, v in bad.items())


def test_check_flags_dead_multiplies(listings):
    res = lds_hazards(listings["planted"])
    flagged = [f for f, v in res.items() if v]
    assert flagged, "a GEMM whose operand reads lost their users was not flagged"
    assert all("gemm_bf16_big8ILi1E" in f for f in flagged), flagged   # only the down projections (EPI_F32)
