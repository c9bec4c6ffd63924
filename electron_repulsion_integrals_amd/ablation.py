"""Ablation harness: variant libraries from the one generator, measured class by class.

"FusionRCG" (section V-B, Ablation Study) generates variant kernel libraries
from the same code generator, toggling one component at a time, and compiles
each as a complete library so that compiler reports and counters reflect the
real code path.  It reports PeakLive and throughput with and without the
axis-priority graph (Fig. 5), with and without DSA scheduling (Fig. 6), with
and without stepwise spherical fusion (Fig. 7), and register-only against
buffered execution over total angular momentum 0..16 (Fig. 8).  This module
does the same for this library's generator (switches in gen/variant.py):

  python -m electron_repulsion_integrals_amd.ablation build [--variants a,b]
      generate and compile every variant library for gfx950 (no GPU needed),
      with the compiler's resource remarks and the generator's graph
      statistics, into electron_repulsion_integrals_amd/ablation_libs/
  python -m electron_repulsion_integrals_amd.ablation run [--variants a,b] [--json F] [--md F]
      time every class of every variant on the GPU, one child process per
      library, and compare every variant's integrals with the full library's

The classes are the diagonal quartets (ab|ab) with total angular momentum
0, 2, ..., 16; inputs are seeded batches of one class with four independent
centres per quartet in a 10-bohr cube, two primitives per shell (exponents
log-uniform in [0.1, 10], coefficients uniform in [0.1, 1]), spherical output.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# (ab|ab) with la + lb + lc + ld = 0, 2, ..., 16
ABLATION_CLASSES = [(0, 0, 0, 0), (1, 0, 1, 0), (1, 1, 1, 1), (2, 1, 2, 1), (2, 2, 2, 2),
                    (3, 2, 3, 2), (3, 3, 3, 3), (4, 3, 4, 3), (4, 4, 4, 4)]
# the lane-tier libraries stop at (fd|fd): beyond it the one-lane graph spills
# tens of kilobytes per lane and takes longer to compile than to be useful
LANE_MAX_L = 10
K_PRIM = 2
SEED = 7000
FP64_PEAK = 78.6e12


def variant_classes(name: str):
    return [c for c in ABLATION_CLASSES if not name.startswith("lane_") or sum(c) <= LANE_MAX_L]


def _tag(ls):
    return "(" + "spdfg"[ls[0]] + "spdfg"[ls[1]] + "|" + "spdfg"[ls[2]] + "spdfg"[ls[3]] + ")"


def _parse_remarks(text: str):
    """{kernel name: {VGPRs, AGPRs, ScratchSize, Occupancy, LDS}} from -Rpass-analysis remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark:\s+Function Name:\s+(\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z \[\]/]+?):\s+(\S+)\s+\[-Rpass", line)
        if m and cur:
            key = m.group(1).strip()
            short = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
                     "Occupancy [waves/SIMD]": "waves_per_simd", "LDS Size [bytes/block]": "lds_bytes"}.get(key)
            if short:
                out[cur][short] = int(m.group(2))
    return out


def graph_stats(ls, topology: str, schedule: str):
    """Nodes, FP64 operations per primitive quartet and PeakLive of the lane-tier
    graph of one class (the whole recurrence of one quartet in one lane)."""
    from .gen import variant, lane as LN, graph as G
    prev = variant.set_variant(variant.Variant(name="stats", topology=topology, schedule=schedule))
    try:
        ci = G.ClassInfo(*ls)
        nodes, targets, ebra, kv, order, base = LN._schedule(ci)
        flops = 0
        for (e, f, m), (kind, ax, dl) in nodes.items():
            if kind == "F":
                continue
            own, other = (e, f) if kind == "b" else (f, e)
            flops += 3 + (4 if own[ax] >= 2 else 0) + (2 if other[ax] > 0 else 0)
        return {"nodes": len(nodes) - len(base), "vrr_flops": flops, "accumulators": len(targets),
                "peak_live": G.peak_live(order, None, base)}
    finally:
        variant.set_variant(prev)


def _tier_name(ci):
    """Tier of the contracted spherical kernel of a class under the current variant."""
    from .gen.emit import tier_of
    from .gen.lane import use_lane_tier
    from .gen.packed import use_packed_contracted
    if tier_of(ci) == "M":
        return "M"
    if use_lane_tier(ci, True):
        return "L"
    return "P" if use_packed_contracted(ci, True) else "V"


def build_all(names, jobs=None):
    from . import build as B
    from .gen import graph as G
    from .gen.emit import tier_of
    from .gen import variant as V
    report = {}
    for name in names:
        classes = [G.ClassInfo(*c) for c in variant_classes(name)]
        remarks = {}
        lib = B.build(variant=name, classes=classes, remarks=remarks, jobs=jobs)
        prev = V.set_variant(name)
        try:
            tiers = {_tag(c): tier_of(G.ClassInfo(*c)) for c in variant_classes(name)}
            tier_names = {_tag(c): _tier_name(G.ClassInfo(*c)) for c in variant_classes(name)}
        finally:
            V.set_variant(prev)
        res = {}
        for fn, text in remarks.items():
            res.update(_parse_remarks(text))
        report[name] = {"variant": V.VARIANTS[name].as_dict(), "library": os.path.relpath(lib, ROOT),
                        "classes": [list(c) for c in variant_classes(name)], "tiers": tiers,
                        "tier_names": tier_names, "resources": res}
        print(f"{name}: {len(res)} kernels", flush=True)
    stats = {}
    for ls in ABLATION_CLASSES:
        if sum(ls) > LANE_MAX_L or sum(ls) == 0:
            continue
        for topo in ("ket_first", "alg1", "bra_first"):
            for sched in ("dsa", "topo"):
                stats[f"{_tag(ls)} {topo} {sched}"] = graph_stats(ls, topo, sched)
    path = os.path.join(PKG, "ablation_libs", "build_report.json")
    old = {}
    if os.path.exists(path):
        with open(path) as f:
            old = json.load(f)
    old.setdefault("variants", {}).update(report)
    old["lane_graph_stats"] = stats
    with open(path, "w") as f:
        json.dump(old, f, indent=1, sort_keys=True)
    return old


def _batch_size(ls):
    from .gen import graph as G
    ci = G.ClassInfo(*ls)
    per_prim, once = G.dag_flops(ci, True)
    per_q = per_prim * K_PRIM ** 4 + once
    # about 3 ms of work at 20% of the FP64 peak, within [2048, 131072] quartets
    return max(2048, min(131072, int(3e-3 * 0.2 * FP64_PEAK / per_q))), per_q


def class_inputs(ls, n):
    sys.path.insert(0, ROOT)
    from workloads.configs import class_batch
    from .gen import graph as G
    cid = G.class_id(*ls)
    return class_batch(SEED + cid, ls, n, K_PRIM, 10.0, 0.1, 10.0)


def measure(name, classes, reps=10, warmup=2, dump=None, nquartets=None):
    """Time every class of one variant library (this process loads only it)."""
    import numpy as np
    import torch
    from . import _lib as E
    from .build import variant_paths, LIB
    E.load(variant_paths(name)[1])
    results = []
    dumps = {}
    for ls in classes:
        n, per_q = _batch_size(ls)
        if nquartets:
            n = nquartets
        sh, q = class_inputs(ls, n)
        print(f"  {name} {_tag(ls)}: {n} quartets", flush=True)
        plan = E.build_quartets(sh, E.ERI_SPHERICAL, q, 0.0)
        out = torch.empty(plan.n_out, dtype=torch.float64, device="cuda")
        s = torch.cuda.current_stream()
        for _ in range(warmup):
            E.compute_batch(plan, out)
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            E.compute_batch(plan, out)
            b.record(s)
            b.synchronize()
            times.append(a.elapsed_time(b))
        times.sort()
        ms = times[len(times) // 2]
        imap = plan.index_map().cpu().numpy()
        blk = plan.n_out // n
        take = min(n, 64)
        got = out[:take * blk].cpu().numpy().reshape(take, blk)
        dumps[_tag(ls)] = (imap[:take, :4].copy(), got)
        results.append({"class": list(ls), "tag": _tag(ls), "quartets": n, "ms": ms, "ms_min": times[0],
                        "ms_max": times[-1], "quartets_per_s": n / (ms * 1e-3),
                        "fp64_frac": n * per_q / (ms * 1e-3) / FP64_PEAK, "algorithmic_flop_per_quartet": per_q})
        plan.close()
        del out
    if dump:
        arrs = {}
        for t, (rows, got) in dumps.items():
            arrs[t + " rows"] = rows
            arrs[t + " out"] = got
        np.savez(dump, **arrs)
    return results


def run_all(names, out_json=None, out_md=None, reps=10, nquartets=None, timeout=900):
    """One child process per variant library (the parent touches no GPU)."""
    import numpy as np
    results = {}
    tmp = tempfile.mkdtemp(prefix="eri_ablation_")
    for name in names:
        dump = os.path.join(tmp, f"{name}.npz")
        js = os.path.join(tmp, f"{name}.json")
        cmd = [sys.executable, "-u", "-m", "electron_repulsion_integrals_amd.ablation", "measure", "--variant", name,
               "--dump", dump, "--json", js, "--reps", str(reps)]
        if nquartets:
            cmd += ["--nquartets", str(nquartets)]
        print(f"variant {name}", flush=True)
        r = subprocess.run(cmd, cwd=ROOT, timeout=timeout)
        if r.returncode != 0:
            raise RuntimeError(f"variant {name} failed with status {r.returncode}")
        with open(js) as f:
            results[name] = json.load(f)
    # every variant's integrals against the full library's, same seeded inputs
    if "full" in names:
        ref = np.load(os.path.join(tmp, "full.npz"))
        for name in names:
            d = np.load(os.path.join(tmp, f"{name}.npz"))
            for row in results[name]:
                t = row["tag"]
                a, b = d[t + " out"], ref[t + " out"]
                assert np.array_equal(d[t + " rows"], ref[t + " rows"])
                row["max_rel_diff_vs_full"] = float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))
    report = {"classes": [list(c) for c in ABLATION_CLASSES], "k_prim": K_PRIM, "results": results}
    bpath = os.path.join(PKG, "ablation_libs", "build_report.json")
    if os.path.exists(bpath):
        with open(bpath) as f:
            report["build"] = json.load(f)
    if out_json:
        with open(out_json, "w") as f:
            json.dump(report, f, indent=1)
    if out_md:
        with open(out_md, "w") as f:
            f.write(markdown(report))
    print(markdown(report), flush=True)
    return report


def markdown(report):
    """Summary tables: time per class, ratios per switched component, agreement
    with the full library, compiler resources and lane-tier graph statistics."""
    res = report["results"]
    names = list(res)
    rows = {}
    for n in names:
        for r in res[n]:
            rows.setdefault(r["tag"], {})[n] = r
    tags = [_tag(c) for c in report["classes"]]
    out = ["Time per batch (median of the timed calls) and algorithmic FP64 fraction of the 78.6 TFLOP/s peak:", "",
           "| class | quartets | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for t in tags:
        cells = []
        for n in names:
            r = rows.get(t, {}).get(n)
            cells.append("—" if r is None else f"{r['ms']:.3f} ms ({100 * r['fp64_frac']:.1f}%)")
        nq = rows.get(t, {}).get(names[0], {}).get("quartets", "")
        out.append(f"| {t} | {nq} | " + " | ".join(cells) + " |")
    pairs = [("no_dsa", "full", "DSA on / off (adaptive tiers)"),
             ("lane_no_dsa", "lane_only", "DSA on / off (lane tier)"),
             ("lane_alg1", "lane_only", "ket-first graph / Algorithm 1 graph (lane tier)"),
             ("lane_bra_first", "lane_only", "ket-first graph / bra-first graph (lane tier)"),
             ("no_sph_fusion", "full", "stepwise fusion / Cartesian then Eq. (17)"),
             ("lane_only", "full", "adaptive / lane tier only"),
             ("memory_only", "full", "adaptive / memory tier only")]
    out += ["", "Speed-up of the first-named configuration (time of the other / time of it):", "",
            "| comparison | " + " | ".join(tags) + " |", "|---|" + "---|" * len(tags)]
    for a, b, label in pairs:
        if a not in names or b not in names:
            continue
        cells = []
        for t in tags:
            ra, rb = rows.get(t, {}).get(a), rows.get(t, {}).get(b)
            cells.append("—" if ra is None or rb is None else f"{ra['ms'] / rb['ms']:.2f}")
        out.append(f"| {label} | " + " | ".join(cells) + " |")
    if any("max_rel_diff_vs_full" in r for n in names for r in res[n]):
        out += ["", "Largest difference from the full library's integrals on the first 64 quartets, relative to the "
                "largest integral of the class:", "", "| variant | " + " | ".join(tags) + " |",
                "|---|" + "---|" * len(tags)]
        for n in names:
            cells = []
            for t in tags:
                r = rows.get(t, {}).get(n)
                cells.append("—" if r is None else f"{r.get('max_rel_diff_vs_full', float('nan')):.1e}")
            out.append(f"| {n} | " + " | ".join(cells) + " |")
    build = report.get("build", {})
    if build.get("variants"):
        out += ["", "Tier of each class (L lane, V lane group in one wave, P packed, M memory):", "",
                "| variant | " + " | ".join(tags) + " |", "|---|" + "---|" * len(tags)]
        for n in names:
            v = build["variants"].get(n)
            if v:
                out.append(f"| {n} | " + " | ".join(v.get("tier_names", v["tiers"]).get(t, "—") for t in tags) + " |")
        out += ["", "Compiler resources of the contracted spherical kernel of each class "
                "(VGPR + AGPR, scratch bytes per lane, waves per SIMD):", "",
                "| variant | " + " | ".join(tags) + " |", "|---|" + "---|" * len(tags)]
        from .gen import graph as G
        for n in names:
            v = build["variants"].get(n)
            if not v:
                continue
            cells = []
            for c in report["classes"]:
                key = f"_Z{len('eri_kernel_c%d_s' % G.class_id(*c))}eri_kernel_c{G.class_id(*c)}_s12EriClassArgs"
                r = v["resources"].get(key)
                cells.append("—" if r is None else
                             f"{r.get('vgpr', 0)}+{r.get('agpr', 0)}, {r.get('scratch_bytes_per_lane', 0)} B, "
                             f"{r.get('waves_per_simd', 0)}")
            out.append(f"| {n} | " + " | ".join(cells) + " |")
    if build.get("lane_graph_stats"):
        st = build["lane_graph_stats"]
        out += ["", "Lane-tier graph of one quartet (generator): recurrence nodes, FP64 operations per primitive "
                "quartet, PeakLive (values, accumulators excluded) under the liveness scheduler / a plain "
                "topological order:", "", "| class | accumulators | ket_first | alg1 | bra_first |", "|---|---|---|---|---|"]
        for t in tags:
            cells = []
            for topo in ("ket_first", "alg1", "bra_first"):
                a, b = st.get(f"{t} {topo} dsa"), st.get(f"{t} {topo} topo")
                if a is None:
                    cells = None
                    break
                cells.append(f"{a['nodes']} nodes, {a['vrr_flops']} FLOP, PeakLive {a['peak_live']} / {b['peak_live']}")
            if cells:
                out.append(f"| {t} | {st[t + ' ket_first dsa']['accumulators']} | " + " | ".join(cells) + " |")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["build", "run", "measure", "md"])
    ap.add_argument("--variants", default=None)
    ap.add_argument("--variant", default=None)
    ap.add_argument("--json", default=None)
    ap.add_argument("--md", default=None)
    ap.add_argument("--dump", default=None)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--nquartets", type=int, default=None)
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    from .gen.variant import VARIANTS
    names = a.variants.split(",") if a.variants else list(VARIANTS)
    if a.what == "build":
        build_all(names, a.jobs)
    elif a.what == "run":
        run_all(names, a.json, a.md, a.reps, a.nquartets)
    elif a.what == "md":
        with open(a.json) as f:
            text = markdown(json.load(f))
        with open(a.md, "w") as f:
            f.write(text)
    else:
        res = measure(a.variant, variant_classes(a.variant), a.reps, dump=a.dump, nquartets=a.nquartets)
        with open(a.json, "w") as f:
            json.dump(res, f)


if __name__ == "__main__":
    main()
