"""Lane tier: one quartet per lane, the whole class in that lane's registers.

For classes with few contracted targets, a lane owns a quartet: it loops over
the quartet's primitive quartets, sets each up itself (geometry and Boys
values: the Gaussian-pair and Boys steps of Algorithm 2 of "FusionRCG"), evaluates
the vertical recurrence of Eq. (2) and its ket twin over every bra component
e at once, adds the targets [e0|f0] into accumulators (as in Algorithm 2),
and after the loop applies the horizontal recurrence of Eq. (3) and the
stepwise spherical transform of Eq. (14) to both pairs.  No value crosses
lanes, so there are no LDS records, no coupling reads and no barriers: the
broadcast of primitive-quartet records that bounds the lane-group tiers by
LDS bandwidth disappears.  This is the page's thread-per-quartet mapping
(section III-C), applied where its live set fits the wave64 register file.

The graph is the one `graph.dag_flops` counts: nodes (e, f, m), bra nodes
(f = 0) raised along the last non-zero axis of e, ket nodes raised along the
axis `build_ket_vrr` chooses, each node evaluated once per primitive quartet;
its order comes from the liveness scheduler.
"""
from __future__ import annotations

from .cartesian import components, sub
from .graph import ClassInfo, build_ket_vrr, build_hrr, class_id, schedule_min_live, peak_live, raise_axis

AX = "xyz"
# accumulators per lane: up to 100 the kernel may drop to one wave per SIMD
# (VGPRs + AGPRs) and is still faster than the lane-group tiers (measured)
MAX_ACC = 100
# bras of total angular momentum 5 or more (56 lanes or more in the lane-group
# tiers, with long per-lane bra paths): up to 200 accumulators (measured on the
# 120-atom cluster: (fd|ps), 138 accumulators, 2.4x faster in this tier, while
# (dp|pp), 144 accumulators and a 20-lane bra, is 8% slower here)
MAX_ACC_WIDE_BRA = 200
MAX_LIVE = 96      # scheduled peak of recurrence values (doubles) besides the accumulators


def _bra_axis(e):
    return 2 if e[2] > 0 else (1 if e[1] > 0 else 0)


def _lowering(e, f, topology):
    """Side ("b" bra, "k" ket) and axis of the raise that produces node (e, f)."""
    if topology == "ket_first":
        if sum(f) > 0:
            return "k", raise_axis(f)  # the ket recurrence's own axis choice
        return "b", _bra_axis(e)
    if topology == "alg1":
        for ax in (2, 1, 0):
            if f[ax] > 0:
                return "k", ax
            if e[ax] > 0:
                return "b", ax
    if topology == "bra_first":
        for side, t in (("b", e), ("k", f)):
            for ax in (0, 1, 2):
                if t[ax] > 0:
                    return side, ax
    raise ValueError(topology)


def lane_vrr(ci: ClassInfo):
    """Nodes {(e, f, m): (kind, axis, deps)} reachable from the targets, and the targets.

    A ket node lowers f along `axis`: operands (e, f-1, m), (e, f-1, m+1), then
    (e, f-2, m), (e, f-2, m+1) when f_axis >= 2, then the coupling operand
    (e-1, f-1, m+1) when e_axis > 0.  A bra node is the mirror image (Eq. (2)).
    """
    from .variant import CURRENT
    kv = build_ket_vrr(ci.lc, ci.Lk)
    ebra = [e for l in range(ci.la, ci.Lb + 1) for e in components(l)]
    targets = [(e, f) for e in ebra for (f, _) in kv.targets]
    nodes = {}
    stack = [(e, f, 0) for (e, f) in targets]
    while stack:
        e, f, m = stack.pop()
        if (e, f, m) in nodes:
            continue
        if sum(e) + sum(f) == 0:
            nodes[(e, f, m)] = ("F", None, [])
            continue
        kind, ax = _lowering(e, f, CURRENT.topology)
        own, other = (f, e) if kind == "k" else (e, f)

        def at(o, t, mm):
            return (t, o, mm) if kind == "k" else (o, t, mm)
        o1 = sub(own, ax)
        deps = [at(o1, other, m), at(o1, other, m + 1)]
        if own[ax] >= 2:
            o2 = sub(own, ax, 2)
            deps += [at(o2, other, m), at(o2, other, m + 1)]
        if other[ax] > 0:
            deps.append(at(o1, sub(other, ax), m + 1))
        nodes[(e, f, m)] = (kind, ax, deps)
        stack += deps
    return nodes, targets, ebra, kv


def _schedule(ci: ClassInfo):
    nodes, targets, ebra, kv = lane_vrr(ci)
    base = [k for k, v in nodes.items() if v[0] == "F"]
    items = [(k, list(v[2]), False) for k, v in nodes.items() if v[0] != "F"]
    for t, (e, f) in enumerate(targets):
        items.append((("acc", t), [(e, f, 0)], True))
    # a topological start order (by total angular momentum, then m descending)
    items.sort(key=lambda it: (0, sum(it[0][0]) + sum(it[0][1]), -it[0][2]) if it[0][0] != "acc" else (1, it[0][1], 0))
    order = schedule_min_live(items, base)
    return nodes, targets, ebra, kv, order, base


def lane_peak(ci: ClassInfo) -> int:
    nodes, targets, ebra, kv, order, base = _schedule(ci)
    return peak_live(order, None, base)


def use_lane_tier(ci: ClassInfo, spherical: bool) -> bool:
    from .variant import CURRENT
    if CURRENT.tiers == "lane":
        return True
    nacc = ci.n_ebra * len(build_ket_vrr(ci.lc, ci.Lk).targets)
    if nacc > (MAX_ACC_WIDE_BRA if ci.Lb >= 5 else MAX_ACC) or ci.L > 7:
        return False
    return lane_peak(ci) <= MAX_LIVE


def emit_lane_tier(ci: ClassInfo, spherical: bool, k1: bool):
    """One kernel per class and output kind (K4 = 1 or any contraction)."""
    from .emit import _hrr_ops, _fmt
    nodes, targets, ebra, kv, order, base = _schedule(ci)
    L = ci.L
    NK = ci.nket(spherical)
    NBO = ci.nbra_out(spherical)
    BLK = ci.nout(spherical)
    cid = class_id(ci.la, ci.lb, ci.lc, ci.ld)
    tag = f"c{cid}_{'s' if spherical else 'c'}" + ("_k1" if k1 else "")
    name = {}
    for k in base:
        name[k] = f"F[{k[2]}]"
    cnt = 0
    for k, v in nodes.items():
        if v[0] != "F":
            name[k] = f"v{cnt}"
            cnt += 1
    o = []
    o.append(f"// one quartet per lane; {len(nodes) - len(base)} recurrence nodes and {len(targets)} accumulators")
    o.append(f"__global__ void __launch_bounds__(64) eri_kernel_{tag}(EriClassArgs a)")
    o.append("{")
    o.append(f"  constexpr int BLK = {BLK};")
    o.append("  const int q0 = blockIdx.x * 64 + threadIdx.x;")
    o.append("  const bool act = q0 < a.nq;")
    o.append("  const int q = act ? q0 : a.nq - 1;")
    o.append("  const int4 pb = a.pair_info[a.qbra[q]], pk = a.pair_info[a.qket[q]];")
    o.append("  const double Ax = a.cen[3 * pb.x], Ay = a.cen[3 * pb.x + 1], Az = a.cen[3 * pb.x + 2];")
    o.append("  const double Cx = a.cen[3 * pk.x], Cy = a.cen[3 * pk.x + 1], Cz = a.cen[3 * pk.x + 2];")
    o.append("  const double ABx = Ax - a.cen[3 * pb.y], ABy = Ay - a.cen[3 * pb.y + 1], ABz = Az - a.cen[3 * pb.y + 2];")
    o.append("  const double CDx = Cx - a.cen[3 * pk.y], CDy = Cy - a.cen[3 * pk.y + 1], CDz = Cz - a.cen[3 * pk.y + 2];")
    o.append("  const double ACx = Ax - Cx, ACy = Ay - Cy, ACz = Az - Cz;")
    o.append("  (void)ABx; (void)ABy; (void)ABz; (void)CDx; (void)CDy; (void)CDz;")
    for t in range(len(targets)):
        o.append(f"  double acc{t} = 0.0;")
    if k1:
        o.append("  {")
        o.append("    const EriPrimPair P = eri_load_pp(a.ppd, pb.z);")
        o.append("    const EriPrimPair K = eri_load_pp(a.ppd, pk.z);")
    else:
        o.append("  for (int ib = 0; ib < pb.w; ++ib) {")
        o.append("  const EriPrimPair P = eri_load_pp(a.ppd, pb.z + ib);")
        o.append("  for (int ik = 0; ik < pk.w; ++ik) {")
        o.append("    const EriPrimPair K = eri_load_pp(a.ppd, pk.z + ik);")
    o.append("    EriQuartetGeom g;")
    o.append("    eri_geom(P, K, ACx, ACy, ACz, g);")
    o.append(f"    double F[{L + 1}];")
    o.append(f"    eri_boys<{L}>(g.T, g.pref, a.boys, F);")
    o.append("    const double PAx = P.PA[0], PAy = P.PA[1], PAz = P.PA[2];")
    o.append("    const double WPx = g.WP[0], WPy = g.WP[1], WPz = g.WP[2];")
    o.append("    const double QCx = K.PA[0], QCy = K.PA[1], QCz = K.PA[2];")
    o.append("    const double WQx = g.WQ[0], WQy = g.WQ[1], WQz = g.WQ[2];")
    o.append("    const double i2z = 0.5 * P.izeta, i2e = 0.5 * K.izeta, roz = g.roz, roe = g.roe, i2ze = g.i2ze;")
    o.append("    (void)PAx; (void)PAy; (void)PAz; (void)WPx; (void)WPy; (void)WPz; (void)QCx; (void)QCy; (void)QCz;")
    o.append("    (void)WQx; (void)WQy; (void)WQz; (void)i2z; (void)i2e; (void)roz; (void)roe; (void)i2ze;")
    tpos = {(e, f): t for t, (e, f) in enumerate(targets)}
    for (k, deps, sink) in order:
        if sink:
            t = k[1]
            e, f = targets[t]
            o.append(f"    acc{t} += {name[(e, f, 0)]};")
            continue
        kind, ax, dl = nodes[k]
        e, f, m = k
        a_ = AX[ax]
        own, other = (e, f) if kind == "b" else (f, e)
        g1, g2, half, ro = ("PA", "WP", "i2z", "roz") if kind == "b" else ("QC", "WQ", "i2e", "roe")
        expr = f"{g1}{a_} * {name[dl[0]]} + {g2}{a_} * {name[dl[1]]}"
        if own[ax] >= 2:
            expr += f" + {_fmt(own[ax] - 1)} * {half} * ({name[dl[2]]} - {ro} * {name[dl[3]]})"
        if other[ax] > 0:
            expr += f" + {_fmt(other[ax])} * i2ze * {name[dl[-1]]}"
        o.append(f"    const double {name[k]} = {expr};")
    o.append("  }")
    if not k1:
        o.append("  }")
    # horizontal recurrences and transforms, ket then bra (Eq. (14): either order), all in this lane
    kops, kbase, kouts = _hrr_ops(ci.lc, ci.ld, "CD", spherical)
    bops, bbase, bouts = _hrr_ops(ci.la, ci.lb, "AB", spherical)
    items, code = [], {}
    nm = {}

    def ref(kk):
        return nm[kk]
    for e in ebra:
        for f in kbase:
            nm[("k", e, ("b", f))] = f"acc{tpos[(e, f)]}"
    ci_ = 0
    for e in ebra:
        for (kk, terms) in kops:
            key = ("k", e, kk)
            nm[key] = f"h{ci_}"
            ci_ += 1
            srcs = [("k", e, s) for _, s in terms]
            items.append((key, [s for s in srcs if not nm[s].startswith("acc")], False))
            code[key] = (key, terms, srcs)
    for ki, ko in enumerate(kouts):
        for e in ebra:
            nm[("b", ki, ("b", e))] = nm[("k", e, ko)]
        for (kk, terms) in bops:
            key = ("b", ki, kk)
            nm[key] = f"h{ci_}"
            ci_ += 1
            srcs = [("b", ki, s) for _, s in terms]
            deps = []
            for s in srcs:
                if s[2][0] == "b":
                    ke = ("k", s[2][1], ko)
                    if not nm[ke].startswith("acc"):
                        deps.append(ke)
                else:
                    deps.append(s)
            items.append((key, deps, False))
            code[key] = (key, terms, srcs)
        for bi, bo in enumerate(bouts):
            src = ("b", ki, bo)
            dep = src if src in code else (("k", bo[1], ko) if bo[0] == "b" else src)
            sk = ("st", bi, ki)
            items.append((sk, [dep] if dep in code else [], True))
            code[sk] = (sk, None, [src])
    for (kk, deps, sink) in schedule_min_live(items, ()):
        key, terms, srcs = code[kk]
        if terms is None:
            bi, ki = kk[1], kk[2]
            o.append(f"  if (act) eri_out_merged(&a.out[(size_t)q * BLK + {bi * NK + ki}], {ref(srcs[0])});")
            continue
        parts = [ref(s) if c is None else f"{c} * {ref(s)}" for (c, _), s in zip(terms, srcs)]
        o.append(f"  const double {nm[key]} = {' + '.join(parts)};")
    o.append("}")
    o.append("")
    o.append(f"void eri_launch_{tag}(const EriClassArgs& a, hipStream_t s)")
    o.append("{")
    o.append("  const int nblk = (a.nq + 63) / 64;")
    o.append(f"  if (nblk > 0) hipLaunchKernelGGL(eri_kernel_{tag}, dim3(nblk), dim3(64), 0, s, a);")
    o.append("}")
    o.append("")
    return o
