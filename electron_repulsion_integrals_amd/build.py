"""Build the HIP library: generate the class kernels, compile for gfx950, link.

Usage: python -m electron_repulsion_integrals_amd.build [--lmax 4] [--jobs N]

Output: electron_repulsion_integrals_amd/liberi_mi355x.so
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
GEN_DIR = os.path.join(CSRC, "generated")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "liberi_mi355x.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed FP32 instructions stay disabled in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", CSRC, "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, use_cache: bool) -> tuple[str, float, str]:
    import time
    with open(src, "rb") as f:
        h = hashlib.sha1(f.read() + " ".join(CFLAGS).encode())
    # headers affect every object
    for hdr in ("eri_device.h", os.path.join("generated", "eri_sph_table.h")):
        if os.path.exists(os.path.join(CSRC, hdr)):
            with open(os.path.join(CSRC, hdr), "rb") as f:
                h.update(f.read())
    with open(os.path.join(ROOT, "include", "eri.h"), "rb") as f:
        h.update(f.read())
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + "." + h.hexdigest()[:16] + ".o")
    if use_cache and os.path.exists(obj):
        return obj, 0.0, ""
    t = time.time()
    tmp = obj + ".tmp.o"
    r = subprocess.run([HIPCC, *CFLAGS, "-c", src, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
    os.replace(tmp, obj)
    return obj, time.time() - t, r.stderr


def build(lmax: int = 4, jobs: int | None = None, use_cache: bool = True, verbose: bool = True) -> str:
    """Generate + compile + link.  ``use_cache`` reuses objects whose source and flags are unchanged."""
    sys.path.insert(0, ROOT)
    from electron_repulsion_integrals_amd.gen.emit import generate
    os.makedirs(OBJ_DIR, exist_ok=True)
    files, entries = generate(GEN_DIR, lmax=lmax)
    keep = {os.path.basename(f) for f in files}
    for fn in os.listdir(GEN_DIR):
        if fn.endswith(".hip") and fn not in keep:
            os.remove(os.path.join(GEN_DIR, fn))
    srcs = [os.path.join(CSRC, "eri_runtime.hip")] + files
    jobs = jobs or min(16, os.cpu_count() or 4)
    objs = [None] * len(srcs)
    # compile the largest sources first so the pool drains evenly
    order = sorted(range(len(srcs)), key=lambda i: -os.path.getsize(srcs[i]))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, srcs[i], use_cache): i for i in order}
        for fu in cf.as_completed(futs):
            i = futs[fu]
            obj, dt, _ = fu.result()
            objs[i] = obj
            if verbose and dt > 20:
                print(f"  compiled {os.path.basename(srcs[i])} in {dt:.0f}s", flush=True)
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} ({len(srcs)} sources, {len(entries)} class kernels)", flush=True)
    return LIB


def resource_report(lmax: int = 4, jobs: int | None = None):
    """Per-kernel VGPR/AGPR/scratch/LDS/occupancy from the compiler's resource remarks."""
    import re
    from electron_repulsion_integrals_amd.gen.emit import generate
    files, entries = generate(GEN_DIR, lmax=lmax)
    jobs = jobs or min(16, os.cpu_count() or 4)

    def one(src):
        r = subprocess.run([HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", os.devnull],
                           capture_output=True, text=True)
        info = {}
        for line in r.stderr.splitlines():
            m = re.search(r"remark:\s+([A-Za-z \[\]/]+?):\s+(\S+)\s+\[-Rpass", line)
            if m:
                info[m.group(1).strip()] = m.group(2)
        return os.path.basename(src), info

    out = {}
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for name, info in ex.map(one, files[:-1]):
            out[name] = info
    return out, entries


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--lmax", type=int, default=4)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--no-cache", action="store_true")
    a = ap.parse_args()
    build(a.lmax, a.jobs, use_cache=not a.no_cache)


if __name__ == "__main__":
    main()
