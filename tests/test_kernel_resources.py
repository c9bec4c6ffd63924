"""Compile-time gate: every class kernel whose shells all have l <= 2 runs without
scratch spills.

"FusionRCG" reports zero register spill for every angular-momentum class up to
a total of 6 in its register tier (section III-C1, Tier 1; section VII).  Here
the l <= 2 classes (total angular momentum up to 8) are generated, compiled for
gfx950 with the compiler's resource remarks, and every kernel of them (the
contracted kernel and the uncontracted one, Cartesian and spherical output) must
report ScratchSize 0.  CPU only: hipcc cross-compiles without a GPU.
"""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from electron_repulsion_integrals_amd import build as B
from electron_repulsion_integrals_amd.gen.emit import generate
from electron_repulsion_integrals_amd.gen.graph import all_classes

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")


def _remarks(src):
    r = subprocess.run([B.HIPCC, *B.CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", os.devnull],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+([A-Za-z \[\]/]+?):\s+(\S+)\s+\[-Rpass", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = kernels.setdefault(val, {})
        elif cur is not None:
            cur[key] = val
    return os.path.basename(src), kernels


def test_l2_class_kernels_have_no_scratch(tmp_path):
    cls = [ci for ci in all_classes(4) if max(ci.la, ci.lb, ci.lc, ci.ld) <= 2]
    assert len(cls) == 21
    files, entries = generate(str(tmp_path), lmax=4, classes=cls)
    srcs = [f for f in files if os.path.basename(f).startswith("eri_c")]
    assert len(srcs) == 42
    spills = []
    n = 0
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
        for name, kernels in ex.map(_remarks, srcs):
            assert kernels, name
            for k, info in kernels.items():
                n += 1
                if int(info["ScratchSize [bytes/lane]"]) != 0:
                    spills.append((name, k, info["ScratchSize [bytes/lane]"], info.get("VGPRs")))
    assert n == 84
    assert not spills, spills
