"""Every kernel instance of libcknv compiles for gfx950 without register
spills: the compiler's resource-usage report gives 0 bytes of scratch per
lane for each. A spill turns a register access into a memory round trip on a
latency-bound path, so it is treated as a build regression. No GPU needed."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from block_sparse_kv_stats_amd import build

HIPCC = next((c for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or "") if c and os.path.exists(c)),
             None)


def _usage(src: str, out_dir: str) -> list:
    cmd = [build.hipcc(), *build.common_flags(), "-c", os.path.join(build.CSRC, src),
           "-o", os.path.join(out_dir, src + ".o"), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    rows, name = [], None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            rows.append((name, int(m.group(1))))
    return rows


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
def test_no_kernel_spills_to_scratch():
    with tempfile.TemporaryDirectory() as d:
        with cf.ThreadPoolExecutor(max_workers=min(6, len(build.SOURCES))) as ex:
            rows = [r for rs in ex.map(lambda s: _usage(s, d), build.SOURCES) for r in rs]
    kernels = [r for r in rows if "kernel" in r[0]]
    assert len(kernels) > 50, f"resource report parsed for only {len(kernels)} kernels"
    spills = [r for r in kernels if r[1] != 0]
    assert not spills, f"kernels using scratch: {spills}"
