"""GPU parity of the ablation variant libraries (electron_repulsion_integrals_amd/ablation.py).

Every variant is a complete library built from the same generator with one
component switched (the lane-tier graph topology, the evaluation order, the
spherical fusion, the tier routing).  Each computes the same integrals, so each
is held to the same bar as the product library: its integrals of every class it
was built for are compared element by element with the oracle, on the seeded
inputs the ablation timings use (first 12 quartets of each class batch, two
primitives per shell, spherical).  The variant runs in a child process of its
own (one library per process).
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from electron_repulsion_integrals_amd import ablation as A
from electron_repulsion_integrals_amd.build import variant_paths
from electron_repulsion_integrals_amd.gen.variant import VARIANTS
from test_gpu_parity import assert_parity

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NQ = 12


def _declared_functions():
    import re
    txt = open(os.path.join(ROOT, "include", "eri.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(eri_[A-Za-z_]+)\s*\(", txt)))


@pytest.mark.parametrize("name", list(VARIANTS))
def test_variant_library_matches_oracle(name, tmp_path):
    lib = variant_paths(name)[1]
    how = "python -m electron_repulsion_integrals_amd.ablation build"
    if not os.path.exists(lib):
        pytest.skip(f"{os.path.relpath(lib, ROOT)} not built ({how})")
    # a variant built before the last change of the C ABI cannot be loaded by the binding
    syms = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True).stdout.split()
    missing = [f for f in _declared_functions() if f not in syms]
    if missing:
        pytest.skip(f"{os.path.relpath(lib, ROOT)} predates the current C ABI (lacks {missing[0]}); rebuild: {how}")
    print(f"case: ablation variant {name}", flush=True)
    dump, js = str(tmp_path / "d.npz"), str(tmp_path / "r.json")
    r = subprocess.run([sys.executable, "-u", "-m", "electron_repulsion_integrals_amd.ablation", "measure",
                        "--variant", name, "--nquartets", str(NQ), "--reps", "1", "--dump", dump, "--json", js],
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, f"variant {name}: child exited with {r.returncode}"
    d = np.load(dump)
    with open(js) as f:
        rows = json.load(f)
    assert [row["class"] for row in rows] == [list(c) for c in A.variant_classes(name)]
    for c in A.variant_classes(name):
        t = A._tag(c)
        sh, q = A.class_inputs(c, NQ)
        imap = d[t + " rows"]
        ref, _ = oracle.eri(sh, imap, True)
        assert_parity(d[t + " out"].ravel(), ref, f"{name} {t}", sh=sh, quartets=imap, spherical=True)
