"""Every gfx950 kernel of the library keeps its per-lane state in registers: no scratch (register
spills or private arrays) and no LDS.

The kernels are HBM streams whose windows, look-ahead rows and dweight partials live in
registers by design.  The compiler may silently move a private array to scratch or, by its
promote-alloca transformation, to LDS when an index stops being a compile-time constant; either
keeps every result right and costs bandwidth (a three-row look-ahead array promoted to LDS made
the backward 10% slower).  This builds the device assembly with the library's own flags and
reads the kernel descriptors.  CPU only: hipcc cross-compiles for gfx950.
"""
import os
import re
import shutil
import subprocess

import pytest

from causal_depthwise_conv1d_width_amd import build

SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")


def _descriptors(text, src):
    kernels = re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S)
    assert kernels, f"no kernels found in {src}"
    out = {}
    for name, body in kernels:
        lds = int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", body).group(1))
        scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body).group(1))
        out[name] = (lds, scratch)
    return out


def test_no_lds_and_no_scratch(tmp_path):
    procs = {}
    for src in SOURCES:  # the sources compile concurrently
        out = tmp_path / (src + ".s")
        cmd = ["hipcc", *build.hipcc_flags(), "-x", "hip", "--cuda-device-only", "-S",
               os.path.join(build.CSRC, src), "-o", str(out)]
        procs[src] = (subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True), out)
    bad = {}
    for src, (proc, out) in procs.items():
        _, err = proc.communicate()
        assert proc.returncode == 0, f"{src}: hipcc failed\n{err}"
        for name, v in _descriptors(out.read_text(), src).items():
            if v != (0, 0):
                bad[name] = v
    assert not bad, f"kernels with (LDS bytes, scratch bytes per lane) != (0, 0): {bad}"
