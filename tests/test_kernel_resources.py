"""Every gfx950 kernel of the library must run without scratch (private)
memory: a kernel that reserves it pays a per-wave set-up at launch and
stack traffic at run time -- typically a device function that was not
inlined or an array indexed at run time.  Compiles each source with the
compiler's resource report (no GPU needed)."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_trainable_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _report(src):
    from block_sparse_trainable_amd.build import CFLAGS, EXTRA
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(os.path.basename(src), []), "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage",
           "-c", src, "-o", os.devnull]
    return subprocess.run(cmd, capture_output=True, text=True).stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_kernel_uses_scratch():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        reports = list(ex.map(_report, srcs))
    bad, seen = [], 0
    for src, rep in zip(srcs, reports):
        name = None
        for line in rep.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
            m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
            if m and name:
                seen += 1
                if int(m.group(1)):
                    bad.append((os.path.basename(src), name, int(m.group(1))))
    assert seen >= 10, "no resource report parsed"
    assert not bad, bad
