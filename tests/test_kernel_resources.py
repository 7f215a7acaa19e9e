"""Build-time check of the HIP kernels for gfx950 (runs on the CPU with hipcc): no kernel
may use scratch memory.  The split kernel runs at 234-256 VGPRs of the 256 a wavefront
gets at two per SIMD; a change that tips it into spilling keeps every result correct but
costs several percent, so it is caught here rather than by timing."""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from factored_rank_kv_amd import build as B


def _compile_remarks(src):
    cmd = [B._hipcc(), *B.HIP_FLAGS, *B.EXTRA_FLAGS.get(os.path.basename(src), []),
           "--cuda-device-only", "-c", src, "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stderr


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="no hipcc")
def test_no_kernel_uses_scratch():
    srcs = B.sources()
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        outs = list(ex.map(_compile_remarks, srcs))
    kernels = 0
    bad = []
    for src, text in zip(srcs, outs):
        name = None
        for line in text.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                continue
            m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
            if m and name:
                kernels += 1
                if int(m.group(1)) != 0:
                    bad.append((os.path.basename(src), name, int(m.group(1))))
    assert kernels >= 10, "no kernel resource remarks parsed"
    assert not bad, f"kernels using scratch: {bad}"
