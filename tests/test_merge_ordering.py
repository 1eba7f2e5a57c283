"""The fused step's cross-part merge, checked in the gfx950 assembly of the
object that build() produced (no GPU needed).

The parts of a unit hand their partial records to the part that completes the
unit's count. Each part stores its record with agent-scope stores
(`global_store ... sc1`, written through to the level every XCD sees), waits
for all of them (`s_waitcnt vmcnt(0)`) and a workgroup barrier, and only
then counts itself in with an atomic add (past 16 parts on its group's
counter, whose last part then counts the group in on the unit's counter:
at most three atomic adds per instance); the completing part reads the
records with agent-scope loads (`... sc1`). The HIP memory model alone does
not order relaxed agent-scope stores before a later relaxed atomic, so the
merge relies on this instruction order; a compiler that moved a store past
the wait or dropped sc1 would break it without any test failing on a
single-XCD path. This test reads the disassembly of every step_kernel
instance and checks the order."""
import os
import re
import shutil
import subprocess

import pytest

from block_sparse_kv_stats_amd import build

LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
STEP_OBJ = os.path.join(build.BUILD_DIR, "step.o")


def _disassembly(tmp):
    fatbin = os.path.join(tmp, "fatbin")
    co = os.path.join(tmp, "step.co")
    subprocess.run([TOOLS[0], f"--dump-section=.hip_fatbin={fatbin}", STEP_OBJ, os.path.join(tmp, "x.o")],
                   check=True, capture_output=True)
    subprocess.run([TOOLS[1], "--unbundle", "--type=o", f"--input={fatbin}",
                    f"--targets=hipv4-amdgcn-amd-amdhsa--{build.ARCH}", f"--output={co}"],
                   check=True, capture_output=True)
    res = subprocess.run([TOOLS[2], "-d", f"--mcpu={build.ARCH}", co], check=True,
                         capture_output=True, text=True)
    return res.stdout


def _functions(dis):
    """{symbol: [instruction text]} for every step_kernel instance."""
    funcs, name = {}, None
    for line in dis.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            name = m.group(1) if "step_kernel" in m.group(1) else None
            if name:
                funcs[name] = []
            continue
        if name and line.startswith("\t"):
            funcs[name].append(line.split("//")[0].strip())
    return funcs


@pytest.mark.skipif(not all(os.path.exists(t) for t in TOOLS), reason="ROCm LLVM tools not found")
@pytest.mark.skipif(not os.path.exists(STEP_OBJ), reason="run __graft_entry__.build() first")
def test_part_records_stored_coherently_and_waited_before_the_count(tmp_path):
    funcs = _functions(_disassembly(str(tmp_path)))
    assert len(funcs) >= 50, f"only {len(funcs)} step_kernel instances found"
    for name, ins in funcs.items():
        # the part counters only: the unit's (up to kFlatParts parts), or a
        # group's and then the unit's; the blocks of the two ways of counting
        # may lie in either order, all after the first one's wait and barrier
        atomics = [i for i, x in enumerate(ins) if x.startswith("global_atomic_add")]
        assert 1 <= len(atomics) <= 3, f"{name}: {len(atomics)} atomic adds"
        at = atomics[0]
        barriers = [i for i, x in enumerate(ins[:at]) if x.startswith("s_barrier")]
        assert len(barriers) >= 3, name
        # the record is written between the barrier that follows the waves'
        # LDS records and the barrier that precedes the count
        window = range(barriers[-3] + 1, at)
        stores = [i for i in window if ins[i].startswith("global_store")]
        assert stores, f"{name}: no record stores before the part counter"
        plain = [ins[i] for i in stores if not re.search(r"\bsc1\b", ins[i])]
        assert not plain, f"{name}: record stores without sc1: {plain[:3]}"
        waits = [i for i in range(stores[-1] + 1, at)
                 if ins[i].startswith("s_waitcnt") and "vmcnt(0)" in ins[i]]
        assert waits, f"{name}: no s_waitcnt vmcnt(0) between the last record store and the counter"
        assert any(ins[i].startswith("s_barrier") for i in range(waits[0], at)), \
            f"{name}: no barrier between the wait and the counter"
        coherent_loads = [x for x in ins if x.startswith("global_load") and re.search(r"\bsc1\b", x)]
        assert len(coherent_loads) >= 3, f"{name}: the merging part's record loads lack sc1"
