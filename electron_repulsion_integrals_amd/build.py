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


def _compile(src: str, use_cache: bool, extra=()) -> tuple[str, float, str]:
    import time
    flags = CFLAGS + list(extra)
    with open(src, "rb") as f:
        h = hashlib.sha1(f.read() + " ".join(flags).encode())
    # headers affect every object
    for hdr in ("eri_device.h", os.path.join("generated", "eri_sph_table.h")):
        if os.path.exists(os.path.join(CSRC, hdr)):
            with open(os.path.join(CSRC, hdr), "rb") as f:
                h.update(f.read())
    with open(os.path.join(ROOT, "include", "eri.h"), "rb") as f:
        h.update(f.read())
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + "." + h.hexdigest()[:16] + ".o")
    if use_cache and os.path.exists(obj):
        err = ""
        if os.path.exists(obj + ".err"):
            with open(obj + ".err") as f:
                err = f.read()
        return obj, 0.0, err
    t = time.time()
    tmp = obj + ".tmp.o"
    r = subprocess.run([HIPCC, *flags, "-c", src, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
    with open(obj + ".err", "w") as f:
        f.write(r.stderr)
    os.replace(tmp, obj)
    return obj, time.time() - t, r.stderr


def variant_paths(name: str):
    """(generated-source directory, library path) of an ablation variant."""
    return (os.path.join(ROOT, "_build", "ablation", name, "generated"),
            os.path.join(PKG, "ablation_libs", f"liberi_{name}.so"))


def build(lmax: int = 4, jobs: int | None = None, use_cache: bool = True, verbose: bool = True,
          variant: str = "full", classes=None, remarks: dict | None = None) -> str:
    """Generate + compile + link.  ``use_cache`` reuses objects whose source and flags are unchanged.

    ``variant`` (gen/variant.py) builds an ablation library of the given
    ``classes`` (all classes by default) from a switched generator into
    ``ablation_libs/``; the default is the product library.  ``remarks``, if
    given, receives the compiler's resource remarks per generated source."""
    sys.path.insert(0, ROOT)
    from electron_repulsion_integrals_amd.gen.emit import generate, sph_table_header, _write_if_changed
    from electron_repulsion_integrals_amd.gen import variant as V
    v = V.VARIANTS[variant]
    product = variant == "full" and classes is None
    gen_dir, lib = (GEN_DIR, LIB) if product else variant_paths(variant)
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    os.makedirs(GEN_DIR, exist_ok=True)
    _write_if_changed(os.path.join(GEN_DIR, "eri_sph_table.h"), sph_table_header())
    from electron_repulsion_integrals_amd.gen.graph import derivative_classes
    prev = V.set_variant(v)
    try:
        # the product library also holds the raised-shell classes of the derivative
        # integrals (Cartesian kernels only); ablation variants leave them out
        files, entries = generate(gen_dir, lmax=lmax, classes=classes,
                                  cartesian_only=derivative_classes(lmax) if product else ())
    finally:
        V.set_variant(prev)
    keep = {os.path.basename(f) for f in files}
    for fn in os.listdir(gen_dir):
        if fn.endswith(".hip") and fn not in keep:
            os.remove(os.path.join(gen_dir, fn))
    srcs = [os.path.join(CSRC, "eri_runtime.hip")] + files
    runtime_extra = [] if v.sph_fusion else ["-DERI_UNFUSED_SPHERICAL"]
    jobs = jobs or min(16, os.cpu_count() or 4)
    objs = [None] * len(srcs)
    # compile the largest sources first so the pool drains evenly
    order = sorted(range(len(srcs)), key=lambda i: -os.path.getsize(srcs[i]))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        kernel_extra = ["-Rpass-analysis=kernel-resource-usage"] if remarks is not None else []
        futs = {ex.submit(_compile, srcs[i], use_cache, runtime_extra if i == 0 else kernel_extra): i for i in order}
        for fu in cf.as_completed(futs):
            i = futs[fu]
            obj, dt, err = fu.result()
            objs[i] = obj
            if remarks is not None and i > 0:
                remarks[os.path.basename(srcs[i])] = err
            if verbose and dt > 20:
                print(f"  compiled {os.path.basename(srcs[i])} in {dt:.0f}s", flush=True)
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} ({len(srcs)} sources, {len(entries)} class kernels)", flush=True)
    return lib


def resource_report(lmax: int = 4, jobs: int | None = None):
    """Per-kernel VGPR/AGPR/scratch/LDS/occupancy from the compiler's resource remarks:
    {source file: {kernel symbol: {remark: value}}}."""
    import re
    from electron_repulsion_integrals_amd.gen.emit import generate
    from electron_repulsion_integrals_amd.gen.graph import derivative_classes
    files, entries = generate(GEN_DIR, lmax=lmax, cartesian_only=derivative_classes(lmax))
    jobs = jobs or min(16, os.cpu_count() or 4)

    def one(src):
        r = subprocess.run([HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", os.devnull],
                           capture_output=True, text=True)
        kernels, info = {}, None
        for line in r.stderr.splitlines():
            m = re.search(r"remark:\s+([A-Za-z \[\]/]+?):\s+(\S+)\s+\[-Rpass", line)
            if m:
                key, val = m.group(1).strip(), m.group(2)
                if key == "Function Name":  # each kernel's remarks start with its name
                    info = kernels.setdefault(val, {})
                if info is not None:
                    info[key] = val
        return os.path.basename(src), kernels

    out = {}
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for name, kernels in ex.map(one, files[:-1]):
            out[name] = kernels
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
