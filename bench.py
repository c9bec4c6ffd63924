"""Benchmark: contracted ERI shell quartets per second on one MI355X, fp64.

Default workload: 20,000 (dd|dd) shell quartets, four independent centres
each, uncontracted, spherical output (625 values per quartet).  A step is one
pass of the integral path over that batch through the C ABI
(eri_compute_batch: primitive-quartet setup, Boys, vertical recurrence,
contraction, horizontal recurrences with the stepwise spherical transform,
output write) with the quartet plan already built and resident in HBM; the
plan build (ingest, normalisation, pair data, sort) is timed once and
reported separately as plan_build_ms.

Prints one JSON line.  Extra keys: per-class throughput and FP64 fraction
for the secondary workloads, the J-build time of the 30-atom cluster, and
the CPU oracle timed on a bounded sample of the default workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP64_VECTOR_PEAK_TFLOPS = 78.6  # 256 CU x 128 FP64 FLOP/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the (dd|dd) K = 1 kernel from two rocprofv3 --pmc
# passes (FETCH_SIZE, WRITE_SIZE in KiB per dispatch), scaled by what the same
# counters read for a 1 GiB device copy (x2.0 and x1.0).  Valid only for the
# kernel sources they were taken on (generated class source and device header):
# reported as null once either changes.
TRAFFIC = {"kernel_sources": ["electron_repulsion_integrals_amd/csrc/generated/eri_c20_s.hip",
                              "electron_repulsion_integrals_amd/csrc/eri_device.h"],
           "sha1": "cdd96791f0cf2aeedced5eab34dbd0b23872fb17",
           "fetch_kib": 4132.99, "fetch_scale": 2.0, "write_kib": 97758.13, "write_scale": 1.0}


def measured_traffic():
    import hashlib
    h = hashlib.sha1()
    try:
        for src in TRAFFIC["kernel_sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    if h.hexdigest() != TRAFFIC["sha1"]:
        return None
    return 1024.0 * (TRAFFIC["fetch_kib"] * TRAFFIC["fetch_scale"] + TRAFFIC["write_kib"] * TRAFFIC["write_scale"])


def _class_flops(plan, spherical):
    """Algorithmic FLOPs of every block of a plan (generator's DAG count)."""
    from electron_repulsion_integrals_amd.gen import graph as G
    per_block = []
    for cid in plan.block_class:
        cid = int(cid)
        la, lb = G.pair_class_ls(_pcb(cid))
        lc, ld = G.pair_class_ls(_pck(cid))
        per_prim, once = G.dag_flops(G.ClassInfo(la, lb, lc, ld), spherical)
        per_block.append((per_prim, once))
    return per_block


def _pcb(cid):
    p = 0
    while (p + 1) * (p + 2) // 2 <= cid:
        p += 1
    return p


def _pck(cid):
    p = _pcb(cid)
    return cid - p * (p + 1) // 2


def time_launches(fn, steps, warmup, stream):
    """Per-call HIP-event times (ms) of fn() on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in ev], wall


def timed_steps(fn, steps, warmup, stream):
    """ms per step of `steps` calls of fn() issued back to back between one pair
    of HIP events on `stream`, with the device synchronized before and after;
    and the host wall time of that region (s)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall


def clock_under_load(fn, seconds=1.0):
    """GPU clocks and power as sysfs reports them while fn() runs back to back for about `seconds`."""
    import threading
    import torch
    box = {}

    def poll():
        time.sleep(seconds / 2)
        box["clocks"] = gpu_clocks()
    th = threading.Thread(target=poll)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(50):
            fn()
        torch.cuda.synchronize()
    th.join()
    return box.get("clocks")


def _read(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def gpu_clocks():
    """Current shader and memory clock levels and average power of the AMD GPUs,
    read in-process from the amdgpu driver's sysfs files (pp_dpm_sclk / pp_dpm_mclk:
    the level marked '*'; hwmon power1_average in microwatts).  None if none is readable."""
    import glob
    cards = {}
    for dev in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        if _read(os.path.join(dev, "vendor")) != "0x1002":
            continue
        info = {}
        for key in ("sclk", "mclk"):
            txt = _read(os.path.join(dev, f"pp_dpm_{key}"))
            if txt:
                cur = [ln.split(":", 1)[1].strip(" *") for ln in txt.splitlines() if ln.rstrip().endswith("*")]
                if cur:
                    info[key] = cur[0]
        for hw in glob.glob(os.path.join(dev, "hwmon", "hwmon*")):
            for fn in ("power1_average", "power1_input"):
                v = _read(os.path.join(hw, fn))
                if v and v.isdigit():
                    info["power_W"] = int(v) / 1e6
                    break
        if info:
            cards[os.path.basename(os.path.dirname(dev))] = info
    return cards or None


PRIM_QMAX = 230.0  # the library's primitive-pair screen of screened plans


def _k4(w, rows):
    """Primitive quartets each quartet (rows of shell indices) evaluates: the
    product of the shells' contraction degrees for an explicit list; for a
    screened list the product of the two shell pairs' kept primitive pairs
    (pairs with alpha beta / (alpha + beta) |AB|^2 <= 230, at least one)."""
    import numpy as np
    rows = np.asarray(rows)[:, :4].astype(np.int64)
    sh = w.shells
    K = np.asarray(sh.nprim, dtype=np.int64)
    if w.quartets is not None:
        return K[rows[:, 0]] * K[rows[:, 1]] * K[rows[:, 2]] * K[rows[:, 3]]
    cen = np.asarray(sh.centers, dtype=np.float64).reshape(-1, 3)
    exps = np.asarray(sh.exps, dtype=np.float64)
    j = np.arange(int(K.max()))
    idx = np.minimum(np.asarray(sh.prim_off, dtype=np.int64)[:len(K), None] + j, len(exps) - 1)
    E = np.where(j < K[:, None], exps[idx], np.nan)

    def kept(a, b):
        d = cen[a] - cen[b]
        ab2 = (d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2]
        al, be = E[a][:, :, None], E[b][:, None, :]
        with np.errstate(invalid="ignore"):
            n = ((al * be) / (al + be) * ab2[:, None, None] <= PRIM_QMAX).sum(axis=(1, 2))
        return np.maximum(n, 1)
    out = np.empty(len(rows), dtype=np.int64)
    for c in range(0, len(rows), 65536):
        r = rows[c:c + 65536]
        out[c:c + 65536] = kept(r[:, 0], r[:, 1]) * kept(r[:, 2], r[:, 3])
    return out


def _block_flops(plan, w, imap):
    """Algorithmic FLOPs per class block: sum over quartets of K4 x per-primitive + once."""
    import numpy as np
    from electron_repulsion_integrals_amd.gen import graph as G
    k4 = _k4(w, imap)
    out = []
    for cid, st, cnt in zip(plan.block_class, plan.block_start, plan.block_count):
        cid, st, cnt = int(cid), int(st), int(cnt)
        pb, pk = _pcb(cid), _pck(cid)
        la, lb = G.pair_class_ls(pb)
        lc, ld = G.pair_class_ls(pk)
        per_prim, once = G.dag_flops(G.ClassInfo(la, lb, lc, ld), w.spherical)
        out.append(int(k4[st:st + cnt].sum()) * per_prim + int(cnt) * once)
    return out


def per_class(E, plan, w, steps, stream):
    """Quartets/s and FP64 fraction of every class block (HIP events per block launch)."""
    import torch
    from electron_repulsion_integrals_amd.gen import graph as G
    imap = plan.index_map().cpu().numpy()
    flops = _block_flops(plan, w, imap)
    out = torch.empty(plan.n_out, dtype=torch.float64, device="cuda")
    res = {}
    for b in range(plan.n_blocks):
        off = int(plan.block_out[b])
        view = out[off:]
        times, _ = time_launches(lambda: E.compute_batch(plan, view, b, b + 1), steps, 1, stream)
        ms = sorted(times)[len(times) // 2]
        la, lb = G.pair_class_ls(_pcb(int(plan.block_class[b])))
        lc, ld = G.pair_class_ls(_pck(int(plan.block_class[b])))
        name = "(" + "spdfg"[la] + "spdfg"[lb] + "|" + "spdfg"[lc] + "spdfg"[ld] + ")"
        tf = flops[b] / (ms * 1e-3) / 1e12
        res[name] = {"quartets": int(plan.block_count[b]), "ms": ms,
                     "quartets_per_s": int(plan.block_count[b]) / (ms * 1e-3),
                     "tflops": tf, "fp64_frac": tf / FP64_VECTOR_PEAK_TFLOPS}
    return res


def j_build(E, w, steps, stream, spherical=True):
    """Screened plan (pairs, Schwarz, sort) + J digestion for a cluster workload."""
    import numpy as np
    import torch
    t0 = time.perf_counter()
    plan = E.build_quartets(w.shells, E.ERI_SPHERICAL if spherical else 0, None, w.tau)
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - t0) * 1e3
    if spherical:
        D = torch.tensor(w.density, device="cuda")
    else:
        # a density of the Cartesian basis, drawn the same way as the spherical one
        rng = np.random.default_rng(1003)
        C = rng.standard_normal((plan.nbf, plan.nbf // 4))
        D = torch.tensor(C @ C.T, device="cuda")
    J = torch.empty_like(D)
    times, _ = time_launches(lambda: E.digest_J(plan, D, J), steps, 1, stream)
    dig = sorted(times)[len(times) // 2]
    K = torch.empty_like(D)
    times, _ = time_launches(lambda: E.digest_JK(plan, D, J, K), steps, 1, stream)
    djk = sorted(times)[len(times) // 2]
    return plan, {"quartets": plan.n_quartets, "class_blocks": plan.n_blocks, "plan_build_ms": plan_ms,
                  "digest_J_ms": dig, "j_build_ms": plan_ms + dig, "digest_JK_ms": djk,
                  "note": "plan_build_ms is host wall time incl. allocation; digest_J_ms and digest_JK_ms "
                          "(J and K in one pass) are HIP-event times"}


def _deriv_flops(w, rows):
    """Algorithmic FLOPs of the auxiliary integrals a derivative call evaluates:
    per slot and centre the class with that shell raised and, for l >= 1,
    lowered (Cartesian kernels), K4 primitive quartets each."""
    import numpy as np
    from electron_repulsion_integrals_amd.gen import graph as G
    rows = np.asarray(rows)
    if len(rows) == 0:
        return 0
    K = np.asarray(w.shells.nprim, dtype=np.int64)
    L = np.asarray(w.shells.l, dtype=np.int64)
    k4 = K[rows[:, 0]] * K[rows[:, 1]] * K[rows[:, 2]] * K[rows[:, 3]]
    l4 = L[rows[:, :4]]
    cache, total = {}, 0
    for p in range(4):
        for dl in (1, -1):
            ll = l4.copy()
            ll[:, p] += dl
            ok = ll[:, p] >= 0
            a, b = np.maximum(ll[:, 0], ll[:, 1]), np.minimum(ll[:, 0], ll[:, 1])
            c, d = np.maximum(ll[:, 2], ll[:, 3]), np.minimum(ll[:, 2], ll[:, 3])
            swap = a * (a + 1) // 2 + b < c * (c + 1) // 2 + d
            key = np.where(swap[:, None], np.stack([c, d, a, b], 1), np.stack([a, b, c, d], 1))
            uk, inv = np.unique(key[ok], axis=0, return_inverse=True)
            for j, kk in enumerate(uk):
                kk = tuple(int(x) for x in kk)
                if kk not in cache:
                    cache[kk] = G.dag_flops(G.ClassInfo(*kk), False)
                per_prim, once = cache[kk]
                sel = inv.ravel() == j
                total += int(k4[ok][sel].sum()) * per_prim + int(sel.sum()) * once
    return total


def deriv_sampled(E, plan, w, per_block=2000):
    """First-derivative integrals (eri_compute_deriv: 12 centre-coordinate blocks
    per quartet) of the first ``per_block`` quartets of every class block of a
    plan; wall time of each call (it builds the auxiliary raised/lowered-shell
    plan, computes those integrals and combines them, then synchronises), and
    the algorithmic FLOPs of the auxiliary integrals over that wall time."""
    import torch
    from electron_repulsion_integrals_amd.gen import graph as G
    res, tot_q, tot_s, tot_f = {}, 0, 0.0, 0
    sph = bool(w.spherical)
    for b in range(plan.n_blocks):
        cid = int(plan.block_class[b])
        la, lb = G.pair_class_ls(_pcb(cid))
        lc, ld = G.pair_class_ls(_pck(cid))
        n = int(min(per_block, plan.block_count[b]))
        first = int(plan.block_start[b])
        nf = (lambda l: 2 * l + 1) if sph else (lambda l: (l + 1) * (l + 2) // 2)
        out = torch.empty(12 * n * nf(la) * nf(lb) * nf(lc) * nf(ld), dtype=torch.float64, device="cuda")
        E.compute_deriv(plan, out, first, n)  # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        E.compute_deriv(plan, out, first, n)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        name = "(" + "spdfg"[la] + "spdfg"[lb] + "|" + "spdfg"[lc] + "spdfg"[ld] + ")"
        fl = _deriv_flops(w, plan.quartets(first, n).cpu().numpy())
        res[name] = {"quartets": n, "ms": dt * 1e3, "quartets_per_s": n / dt,
                     "aux_tflops": fl / dt / 1e12, "fp64_frac": fl / dt / 1e12 / FP64_VECTOR_PEAK_TFLOPS}
        tot_q += n
        tot_s += dt
        tot_f += fl
    return {"quartets": tot_q, "seconds": tot_s, "quartets_per_s": tot_q / tot_s if tot_s else None,
            "aux_tflops": tot_f / tot_s / 1e12 if tot_s else None,
            "fp64_frac": tot_f / tot_s / 1e12 / FP64_VECTOR_PEAK_TFLOPS if tot_s else None,
            "note": "wall time per call, including the auxiliary plan build and the host read-back of the "
                    "slots; FLOPs are the auxiliary integrals' algorithmic count; 12 derivative blocks per quartet",
            "per_class": res}


def c5_sampled(E, w, stream, strata=8, max_doubles=1.5e8, max_quartets=1000000):
    """The 120-atom cluster: the full screened plan (implicit) is built and
    timed; every class block is then sampled in ``strata`` evenly spaced
    slot ranges (blocks are ordered by contraction length, so the strata span
    the block's K mix) and timed with HIP events.  The full integral time is
    extrapolated block by block -- an estimate, labelled as such: evaluating
    all 2e10 quartets takes about an hour (c5_measured times it piece by
    piece).  A stratum of a one-quartet-per-lane class holds up to 125,000
    quartets: smaller launches leave most of the GPU idle and would make the
    estimate pessimistic."""
    import numpy as np
    import torch
    from electron_repulsion_integrals_amd.gen import graph as G
    t0 = time.perf_counter()
    plan = E.build_quartets(w.shells, E.ERI_SPHERICAL, None, w.tau)
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - t0) * 1e3
    classes, est_total_s, flops_total, sample_s = {}, 0.0, 0.0, 0.0
    for b in range(plan.n_blocks):
        cid, cnt = int(plan.block_class[b]), int(plan.block_count[b])
        la, lb = G.pair_class_ls(_pcb(cid))
        lc, ld = G.pair_class_ls(_pck(cid))
        ci = G.ClassInfo(la, lb, lc, ld)
        blk = ci.nout(True)
        m = int(min(cnt, max_quartets, max(strata, max_doubles // blk)))
        per = max(1, m // strata)
        firsts = [int(x) for x in np.linspace(0, cnt - per, strata).astype(np.int64)]
        out = torch.empty(per * blk, dtype=torch.float64, device="cuda")
        ms, flops = 0.0, 0.0
        per_prim, once = G.dag_flops(ci, True)
        for f in firsts:
            times, _ = time_launches(lambda: E.compute_range(plan, b, f, per, out), 3, 1, stream)
            ms += sorted(times)[1]
            rows = plan.quartets(int(plan.block_start[b]) + f, per).cpu().numpy()
            k4 = _k4(w, rows)
            flops += float(k4.sum()) * per_prim + per * once
        n = per * len(firsts)
        est_s = ms * 1e-3 * cnt / n
        est_total_s += est_s
        flops_total += flops * cnt / n
        sample_s += ms * 1e-3
        name = "(" + "spdfg"[la] + "spdfg"[lb] + "|" + "spdfg"[lc] + "spdfg"[ld] + ")"
        classes[name] = {"quartets": cnt, "sampled": n, "sample_ms": ms, "quartets_per_s": n / (ms * 1e-3),
                         "tflops": flops / (ms * 1e-3) / 1e12,
                         "fp64_frac": flops / (ms * 1e-3) / 1e12 / FP64_VECTOR_PEAK_TFLOPS}
    return {"quartets": plan.n_quartets, "class_blocks": plan.n_blocks, "plan_build_ms": plan_ms,
            "estimated_integral_s": est_total_s,
            "estimated_fp64_frac": flops_total / est_total_s / 1e12 / FP64_VECTOR_PEAK_TFLOPS,
            "note": "plan built and timed in full; integrals timed on 8 evenly spaced slot ranges per class block "
                    "and extrapolated per block (estimate, not a measured J build)",
            "per_class": classes}


def cpu_baseline(w, seconds=12.0):
    """The oracle as it stands on a bounded prefix of the workload's quartets."""
    import numpy as np
    import oracle
    q = np.asarray(w.quartets)
    done, t_used, n = 0, 0.0, 256
    while t_used < seconds:
        sel = q[np.arange(done, done + n) % len(q)]
        t0 = time.perf_counter()
        oracle.eri(w.shells, sel, w.spherical)
        t_used += time.perf_counter() - t0
        done += n
        n = min(4 * n, 1 << 16)
    return {"value": done / t_used, "unit": "shell quartets/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} quartets of the default workload (cycling its {len(q)} quartets), {t_used:.1f} s"}


def cpu_baselines_per_config(seconds=6.0):
    """The oracle (OpenMP on the host cores) on the other configurations, per
    class: the tiny molecule in full; the (ff|ff) and (gg|gg) batches and the
    30-atom cluster's screened quartets on bounded seeded samples (about
    ``seconds`` each), the cluster's full-J oracle time extrapolated from its
    sample (an estimate, labelled as such)."""
    import numpy as np
    import oracle
    from oracle import plan as oplan
    from workloads import make_config
    res = {"cores": oracle.num_threads()}

    def timed(sh, q, sph):
        t0 = time.perf_counter()
        oracle.eri(sh, q, sph)
        return time.perf_counter() - t0

    w1 = make_config(1)
    q1 = np.array([(i, j, k, l) for i in range(8) for j in range(i + 1) for k in range(8) for l in range(k + 1)
                   if i * (i + 1) // 2 + j >= k * (k + 1) // 2 + l])
    dt = timed(w1.shells, q1, False)
    res["tiny_molecule_cartesian"] = {"quartets": len(q1), "seconds": dt, "quartets_per_s": len(q1) / dt}
    w4 = make_config(4)
    for name, sl in (("(ff|ff)", slice(0, 4000)), ("(gg|gg)", slice(4000, 5000))):
        q = np.asarray(w4.quartets)[sl]
        n, used = 16, 0.0
        while True:
            dt = timed(w4.shells, q[:n], True)
            if dt > seconds / 4 or n >= len(q):
                break
            n = min(len(q), n * 4)
        res[name + " K=2 spherical"] = {"quartets": n, "seconds": dt, "quartets_per_s": n / dt,
                                        "sample": f"first {n} of {len(q)} quartets"}
    w3 = make_config(3)
    S = oracle.schwarz(w3.shells, True)
    p3 = oplan.screened_plan(w3.shells.l, w3.shells.nprim, S, w3.tau)
    q3 = p3["index_map"][:, :4]
    rng = np.random.default_rng(3)
    n = 4096
    while True:
        sel = q3[rng.choice(len(q3), n, replace=False)]
        dt = timed(w3.shells, sel, True)
        if dt > seconds / 2 or n * 4 > len(q3):
            break
        n *= 4
    res["30-atom SVP-like cluster"] = {"quartets": n, "seconds": dt, "quartets_per_s": n / dt,
                                       "sample": f"{n} seeded quartets of its {len(q3)} screened quartets",
                                       "full_J_integrals_estimated_s": dt * len(q3) / n}
    return res


def c5_pieces(E, plan, w, n_target=400, setup_flops=150, samples=64):
    """The 120-atom cluster's J build cut into about ``n_target`` slot ranges
    (block, first, count) of similar estimated cost, in block order.  A block's
    cost per slot is estimated from K4 at ``samples`` evenly spaced slots
    (blocks are ordered by contraction length): per primitive quartet the
    graph's FLOPs plus ``setup_flops`` for its set-up, plus the per-quartet
    part.  Deterministic for a given plan."""
    import numpy as np
    from electron_repulsion_integrals_amd.gen import graph as G
    blocks = []
    for b in range(plan.n_blocks):
        cid, st, cnt = int(plan.block_class[b]), int(plan.block_start[b]), int(plan.block_count[b])
        la, lb = G.pair_class_ls(_pcb(cid))
        lc, ld = G.pair_class_ls(_pck(cid))
        per_prim, once = G.dag_flops(G.ClassInfo(la, lb, lc, ld), True)
        pos = np.unique(np.linspace(0, cnt - 1, min(cnt, samples)).astype(np.int64))
        rows = np.concatenate([plan.quartets(st + int(p_), 1).cpu().numpy() for p_ in pos])
        cost_at = (per_prim + setup_flops) * _k4(w, rows).astype(np.float64) + once
        # cumulative cost at every sample position, trapezoid between them
        cum = np.concatenate([[0.0], np.cumsum(0.5 * (cost_at[1:] + cost_at[:-1]) * np.diff(pos))])
        total = cum[-1] + cost_at[-1]
        blocks.append((b, cnt, pos, cum, total))
    grand = sum(t for *_, t in blocks)
    cap = grand / n_target
    pieces = []
    for b, cnt, pos, cum, total in blocks:
        npc = max(1, int(np.ceil(total / cap)))
        cuts = [0]
        for k in range(1, npc):
            cuts.append(int(np.interp(total * k / npc, cum, pos)))
        cuts.append(cnt)
        cuts = sorted(set(cuts))
        for f, g in zip(cuts, cuts[1:]):
            pieces.append((b, f, g - f))
    return pieces, grand


def c5_measured(E, first_piece, last_piece, budget_s, stream):
    """Measured J build of the 120-atom cluster, slot range by slot range
    (eri_digest_J_range into one J): pieces [first_piece, last_piece) of
    c5_pieces, each timed with HIP events, one JSON line per piece; stops
    before a piece once ``budget_s`` of wall time has passed.  The last line
    carries the totals and sampled elements of this run's partial J (the
    partial J of all runs add up to the full J)."""
    import numpy as np
    import torch
    from workloads import make_config
    from electron_repulsion_integrals_amd.gen import graph as G
    t_start = time.perf_counter()
    w = make_config(5)
    t0 = time.perf_counter()
    plan = E.build_quartets(w.shells, E.ERI_SPHERICAL, None, w.tau)
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - t0) * 1e3
    pieces, grand = c5_pieces(E, plan, w)
    last_piece = min(last_piece, len(pieces))
    D = torch.tensor(w.density, device="cuda")
    J = torch.zeros_like(D)
    print(json.dumps({"c5_pieces": len(pieces), "plan_build_ms": plan_ms, "quartets": plan.n_quartets,
                      "first_piece": first_piece}), flush=True)
    done_ms, nq, i = 0.0, 0, first_piece
    while i < last_piece:
        if time.perf_counter() - t_start > budget_s:
            break
        b, f, n = pieces[i]
        a_, z_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        E.digest_J_range(plan, b, f, n, D, J)
        z_.record(stream)
        z_.synchronize()
        ms = a_.elapsed_time(z_)
        done_ms += ms
        nq += n
        cid = int(plan.block_class[b])
        la, lb = G.pair_class_ls(_pcb(cid))
        lc, ld = G.pair_class_ls(_pck(cid))
        name = "(" + "spdfg"[la] + "spdfg"[lb] + "|" + "spdfg"[lc] + "spdfg"[ld] + ")"
        print(json.dumps({"piece": i, "block": b, "class": name, "first": f, "count": n, "ms": ms}), flush=True)
        i += 1
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    nbf = D.shape[0]
    idx = rng.integers(0, nbf, size=(256, 2))
    Jh = J.cpu().numpy()
    print(json.dumps({"c5_part_done": True, "pieces": [first_piece, i], "next_piece": i, "of": len(pieces),
                      "quartets": nq, "digest_ms": done_ms, "J_sum": float(Jh.sum()),
                      "J_abs_sum": float(np.abs(Jh).sum()), "J_trace": float(np.trace(Jh)),
                      "J_asym_max": float(np.abs(Jh - Jh.T).max()),
                      "J_samples": [[int(r), int(c), float(Jh[r, c])] for r, c in idx]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary workloads and the extra launches (back to back, clocks, FMA rate)")
    ap.add_argument("--only-j-build", action="store_true",
                    help="only the 30-atom cluster: J build and per-class times (for profiler runs)")
    ap.add_argument("--c5-j-pieces", default="",
                    help="A:B -- measured 120-atom J build, slot-range pieces A..B-1 (see c5_pieces)")
    ap.add_argument("--budget-s", type=float, default=900.0,
                    help="with --c5-j-pieces: start no piece after this many seconds")
    ap.add_argument("--only-deriv", action="store_true",
                    help="only the 30-atom cluster's first derivatives, 50,000 slots per class block (profiler runs)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run one plain device copy of this many MiB (scales rocprofv3 FETCH/WRITE_SIZE)")
    a = ap.parse_args()
    if a.calibrate_copy_mib:
        import torch
        n = a.calibrate_copy_mib * (1 << 20) // 8
        src = torch.ones(n, dtype=torch.float64, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_MiB": a.calibrate_copy_mib}), flush=True)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (one process, one MI355X).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import electron_repulsion_integrals_amd as E
    from workloads import make_config

    E.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if a.c5_j_pieces:
        lo, hi = (int(x) for x in a.c5_j_pieces.split(":"))
        c5_measured(E, lo, hi, a.budget_s, stream)
        return
    if a.only_deriv:
        w3 = make_config(3)
        plan3 = E.build_quartets(w3.shells, E.ERI_SPHERICAL, None, w3.tau)
        print(json.dumps({"derivatives_30atom_svp_50k": deriv_sampled(E, plan3, w3, per_block=50000)}), flush=True)
        return
    if a.only_j_build:
        w3 = make_config(3)
        plan3, jb = j_build(E, w3, 5, stream)
        print(json.dumps({"j_build_30atom_svp": jb, "per_class": per_class(E, plan3, w3, 3, stream)}), flush=True)
        return
    w = make_config(2)
    t0 = time.perf_counter()
    plan = E.build_quartets(w.shells, E.ERI_SPHERICAL, w.quartets, 0.0)
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - t0) * 1e3
    out = torch.empty(plan.n_out, dtype=torch.float64, device="cuda")
    # the timed region: K steps back to back, the device synchronized on both sides
    ms, wall = timed_steps(lambda: E.compute_batch(plan, out), a.steps, a.warmup, stream)
    # single launches between their own events, for the spread (each includes the launch gap)
    times, _ = time_launches(lambda: E.compute_batch(plan, out), a.steps, 0, stream)
    clocks = fma_tflops = None
    if not a.no_extra:  # extra launches would also enter a profiler's per-kernel average
        clocks = clock_under_load(lambda: E.compute_batch(plan, out))
        fma_tflops = E.fp64_fma_tflops()
    nq = plan.n_quartets
    (per_prim, once), = _class_flops(plan, True)
    flops = nq * (per_prim + once)  # K = 1: one primitive quartet per quartet
    achieved = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "contracted ERI shell-quartets/sec per L-class + % FP64 peak; J-build time",
        "value": nq / (ms * 1e-3),
        "unit": "shell quartets/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "(dd|dd) x 20000, 4 independent centres in a 10-bohr cube, K=1, "
                               "exponents log-uniform [0.05, 20], spherical output, seed 1002",
                   "quartets": nq, "output_doubles": plan.n_out},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": FP64_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP64_VECTOR_PEAK_TFLOPS, "traffic": measured_traffic()},
        "ms_single_launch_median": sorted(times)[len(times) // 2],
        "ms_single_launch_min": min(times),
        "ms_single_launch_max": max(times),
        "gpu_clocks_under_load": clocks,
        "fp64_fma_measured_TFLOPs": fma_tflops,
        "achieved_over_measured_fma": achieved / fma_tflops if fma_tflops else None,
        "output_write_GBps": plan.n_out * 8 / (ms * 1e-3) / 1e9,
        "plan_build_ms": plan_ms,
        "wall_s_timed_region": wall,
    }
    if not a.no_extra:
        res["per_class"] = {}
        res["per_class"]["(dd|dd) x 20000"] = per_class(E, plan, w, 10, stream)
        w3 = make_config(3)
        plan3, jb = j_build(E, w3, 5, stream)
        res["j_build_30atom_svp"] = jb
        plan3c, jbc = j_build(E, w3, 5, stream, spherical=False)
        del plan3c
        res["j_build_30atom_svp_cartesian"] = jbc
        res["per_class"]["30-atom SVP-like cluster"] = per_class(E, plan3, w3, 3, stream)
        res["derivatives_30atom_svp"] = deriv_sampled(E, plan3, w3)
        res["derivatives_30atom_svp_50k"] = deriv_sampled(E, plan3, w3, per_block=50000)
        del plan3
        w4 = make_config(4)
        plan4 = E.build_quartets(w4.shells, E.ERI_SPHERICAL, w4.quartets, 0.0)
        res["per_class"]["(ff|ff) x 4000 + (gg|gg) x 1000"] = per_class(E, plan4, w4, 3, stream)
        del plan4
        res["c5_120atom_tzvp"] = c5_sampled(E, make_config(5), stream)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w)
        if not a.no_extra:
            res["cpu_baseline_per_config"] = cpu_baselines_per_config()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
