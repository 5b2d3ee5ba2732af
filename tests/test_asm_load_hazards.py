"""The kernels' inline-assembly load blocks, checked on the built gfx950 code
(CPU only: hipcc cross-compiles).

A block of several loads written in assembly reads its address registers
at each load's issue, while the earlier loads of the block may already have
written their destinations.  If the compiler placed a destination on top of
an address that a later load of the block uses, that load could read from
a wrong address; early-clobber outputs forbid it.  This test compiles every
HIP source with the library's flags, walks each assembly block of the
generated code and fails if a load's address register was the destination
of an earlier load in the same block."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from long_context_decode_kvq_amd import build as B

LOADS = ("ds_read", "global_load", "buffer_load", "scratch_load", "flat_load")


def _regs(tok: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def overlapping_blocks(asm: str):
    """Assembly blocks in which a load reads an address register that an
    earlier load of the same block writes."""
    bad, block, in_block = [], [], False
    for line in asm.splitlines():
        if ";;#ASMSTART" in line:
            in_block, block = True, []
            continue
        if ";;#ASMEND" in line:
            written = set()
            for ins in block:
                op, _, rest = ins.partition(" ")
                if not op.startswith(LOADS):
                    continue
                ops = [o.strip() for o in rest.split(",")]
                addr = ops[1].split()[0] if len(ops) > 1 and ops[1] else ""
                if _regs(addr) & written:
                    bad.append(block)
                    break
                if op.startswith(LOADS) and not op.startswith(("global_load_lds", "buffer_load_lds")):
                    written |= _regs(ops[0])
            in_block = False
            continue
        if in_block:
            block.append(line.strip())
    return bad


def test_checker_catches_an_overlap():
    asm = ";;#ASMSTART\nds_read_b64 v[4:5], v5\nds_read_u16 v9, v4 offset:96\n;;#ASMEND\n"
    assert overlapping_blocks(asm)
    ok = ";;#ASMSTART\nds_read_b64 v[6:7], v5\nds_read_u16 v9, v4 offset:96\n;;#ASMEND\n"
    assert not overlapping_blocks(ok)


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="needs hipcc")
def test_no_load_destination_overlaps_a_later_address(tmp_path):
    srcs = sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip"))

    def compile_one(f):
        out = str(tmp_path / (f + ".s"))
        cmd = [B.HIPCC, *B.HIP_FLAGS, "-S", "--offload-device-only",
               os.path.join(B.CSRC, f), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return f, open(out).read()

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(compile_one, srcs))
    n_blocks = 0
    for f, asm in results:
        n_blocks += asm.count(";;#ASMSTART")
        bad = overlapping_blocks(asm)
        assert not bad, f"{f}: {bad[0]}"
    assert n_blocks > 0
