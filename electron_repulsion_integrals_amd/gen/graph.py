"""Recurrence graphs for one angular-momentum class and their schedules.

"FusionRCG" (section II-A) evaluates (ab|cd) in two phases: the vertical
recurrence Eq. (2) builds [e0|f0]^(m) from the Boys values, the contraction of
Algorithm 2 sums them over primitive quartets, and the horizontal recurrence
Eq. (3) moves angular momentum onto the second centre of each pair.  Section
III-A observes that the choice of the axis raised at each node changes the
graph, and that the evaluation order changes how many values are live at once
(PeakLive, Eq. (4)).

Mapping used by the library (wave64-native, not the page's thread per quartet):
every lane of a lane group owns one bra component e (|e| <= la+lb).  A lane
first walks its own path from [00|00]^(m) to [e0|00]^(m) (bra phase), then runs
the ket phase of Eq. (2) -- raising f one unit at a time, the "ket twin" of the
printed bra formula -- as straight-line code over nodes (f, m).  The only
operand owned by another lane is the coupling term [e-1_i 0|f-1_i 0]^(m+1),
which is fetched from lane e-1_i of the same group.

This module builds those graphs, chooses the raise axis per node, orders the
nodes, and measures the resulting peak liveness; emit.py turns them into HIP.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from .cartesian import components, components_upto, sub, add, ncart, nsph, sph_matrix

# Axis priority within one side: z first, then y, then x ("FusionRCG" section
# III-A, Algorithm 1 visits z before y before x for the consumer side).
AXIS_PRIORITY = (2, 1, 0)


def raise_axis(t):
    for ax in AXIS_PRIORITY:
        if t[ax] > 0:
            return ax
    raise ValueError("no axis to lower for the zero triple")


@dataclass
class KetNode:
    f: tuple
    m: int
    axis: int
    a0: tuple  # (f-1i, m)
    a1: tuple  # (f-1i, m+1) -- also the coupling source in lane e-1i
    b0: tuple | None  # (f-2i, m)
    b1: tuple | None  # (f-2i, m+1)
    fi_minus_1: int  # f_i - 1 (coefficient of the 1/(2 eta) term)


@dataclass
class KetVRR:
    lc: int
    Lk: int
    nodes: list = field(default_factory=list)  # KetNode in evaluation order
    base_m: int = 0  # highest m needed from the bra phase at f = 0
    targets: list = field(default_factory=list)  # (f, 0) with |f| in [lc, Lk]


def build_ket_vrr(lc: int, Lk: int, order: str = "level") -> KetVRR:
    """Closure of the targets [e0|f0]^(0), |f| in [lc, Lk], under the ket raise."""
    targets = [(f, 0) for l in range(lc, Lk + 1) for f in components(l)]
    needed = {}
    stack = [t for t in targets if sum(t[0]) > 0]
    base_m = 0 if any(sum(t[0]) == 0 for t in targets) else -1
    while stack:
        f, m = stack.pop()
        if (f, m) in needed:
            continue
        ax = raise_axis(f)
        f1 = sub(f, ax)
        a0, a1 = (f1, m), (f1, m + 1)
        b0 = b1 = None
        if f[ax] >= 2:
            f2 = sub(f, ax, 2)
            b0, b1 = (f2, m), (f2, m + 1)
        needed[(f, m)] = KetNode(f, m, ax, a0, a1, b0, b1, f[ax] - 1)
        for p in (a0, a1, b0, b1):
            if p is None:
                continue
            if sum(p[0]) == 0:
                base_m = max(base_m, p[1])
            elif p not in needed:
                stack.append(p)
    allf = components_upto(Lk)
    fpos = {f: i for i, f in enumerate(allf)}
    nodes = list(needed.values())
    if order == "level":
        nodes.sort(key=lambda n: (sum(n.f), fpos[n.f], n.m))
    else:
        raise ValueError(order)
    return KetVRR(lc, Lk, nodes, max(base_m, 0), targets)


def ket_vrr_peak_live(kv: KetVRR) -> int:
    """Peak number of simultaneously live ket-phase values (base values included)."""
    last = {}
    for t, n in enumerate(kv.nodes):
        for p in (n.a0, n.a1, n.b0, n.b1):
            if p is not None:
                last[p] = t
    for tgt in kv.targets:
        last[tgt] = len(kv.nodes)  # accumulated after the node loop... conservatively
    live = {((0, 0, 0), m) for m in range(kv.base_m + 1)}
    peak = len(live)
    for t, n in enumerate(kv.nodes):
        live.add((n.f, n.m))
        peak = max(peak, len(live))
        for p in (n.a0, n.a1, n.b0, n.b1):
            if p is not None and last.get(p, -1) == t and p not in kv.targets:
                live.discard(p)
        # targets are consumed (accumulated) right after they are produced
        if (n.f, n.m) in kv.targets and last.get((n.f, n.m), -1) <= t:
            live.discard((n.f, n.m))
    return peak


@dataclass
class HRRNode:
    x: tuple
    y: tuple
    axis: int
    p_hi: tuple  # (x+1i, y-1i)
    p_lo: tuple  # (x, y-1i)


def build_hrr(l1: int, l2: int):
    """(x, y+1_i) = (x+1_i, y) + R_i (x, y), Eq. (3), for |x| = l1, |y| = l2.

    Returns (nodes in evaluation order, base triples e with |e| in [l1, l1+l2]).
    Base values are (e, 0).
    """
    need = {}

    def visit(x, y):
        if sum(y) == 0 or (x, y) in need:
            return
        ax = raise_axis(y)
        y1 = sub(y, ax)
        hi = (add(x, ax), y1)
        lo = (x, y1)
        visit(*hi)
        visit(*lo)
        need[(x, y)] = HRRNode(x, y, ax, hi, lo)

    for x in components(l1):
        for y in components(l2):
            visit(x, y)
    nodes = sorted(need.values(), key=lambda n: (sum(n.y), -sum(n.x), n.x, n.y))
    base = [e for l in range(l1, l1 + l2 + 1) for e in components(l)]
    return nodes, base


def transform_terms(l: int):
    """Non-zero (m_index, [(cart_index, coef)]) rows of t^(l)."""
    T = sph_matrix(l)
    return [[(c, v) for c, v in enumerate(row) if v != 0.0] for row in T]


@dataclass
class ClassInfo:
    la: int
    lb: int
    lc: int
    ld: int

    @property
    def Lb(self):
        return self.la + self.lb

    @property
    def Lk(self):
        return self.lc + self.ld

    @property
    def L(self):
        return self.Lb + self.Lk

    @property
    def lanes(self):
        return components_upto(self.Lb)

    @property
    def G(self):
        return len(self.lanes)

    def nout(self, spherical):
        f = nsph if spherical else ncart
        return f(self.la) * f(self.lb) * f(self.lc) * f(self.ld)

    def nket(self, spherical):
        f = nsph if spherical else ncart
        return f(self.lc) * f(self.ld)

    def nbra_out(self, spherical):
        f = nsph if spherical else ncart
        return f(self.la) * f(self.lb)

    @property
    def n_ebra(self):
        return sum(ncart(l) for l in range(self.la, self.Lb + 1))

    @property
    def e_bra_offset(self):
        return sum(ncart(l) for l in range(0, self.la))


def pair_class(la, lb):
    la, lb = max(la, lb), min(la, lb)
    return la * (la + 1) // 2 + lb


def pair_class_ls(pc):
    la = 0
    while (la + 1) * (la + 2) // 2 <= pc:
        la += 1
    return la, pc - la * (la + 1) // 2


def class_id(la, lb, lc, ld):
    pb, pk = pair_class(la, lb), pair_class(lc, ld)
    assert pb >= pk
    return pb * (pb + 1) // 2 + pk


def all_classes(lmax: int = 4):
    out = []
    for pb in range((lmax + 1) * (lmax + 2) // 2):
        for pk in range(pb + 1):
            la, lb = pair_class_ls(pb)
            lc, ld = pair_class_ls(pk)
            out.append(ClassInfo(la, lb, lc, ld))
    return out


def derivative_classes(lmax: int = 4):
    """Classes with one shell raised to l = lmax + 1 and the others at most lmax:
    the neighbouring classes a first derivative with respect to a centre needs
    (d/dA_i phi_a = 2 alpha phi_(a+1_i) - a_i phi_(a-1_i)) when the differentiated
    shell has l = lmax.  Canonical form: bra (lmax+1, lb), lb <= lmax, any ket
    pair of shells up to lmax."""
    out = []
    for lb in range(lmax + 1):
        for pk in range((lmax + 1) * (lmax + 2) // 2):
            lc, ld = pair_class_ls(pk)
            out.append(ClassInfo(lmax + 1, lb, lc, ld))
    return out


def flop_count(ci: ClassInfo, spherical: bool, K4: int = 1):
    """Algorithmic FP64 operations (one FMA = 2) of the generated algorithm per quartet.

    Counts the ket phase for every lane that produces a needed value, the bra
    phase paths, the accumulation, both HRR phases and the transforms.  Boys
    and the pair geometry are counted as a fixed 60 operations per primitive
    quartet.
    """
    kv = build_ket_vrr(ci.lc, ci.Lk)
    per_prim = 0
    # bra phase: each lane e walks |e| steps, step s produces L-s+1 values at 4 flops + 3
    for e in ci.lanes:
        for s in range(1, sum(e) + 1):
            per_prim += (ci.L - s + 1) * 4
    # ket phase: 2 (QC, WQ) + 2 (coupling) + 3 (f_i-1 term) per node
    for n in kv.nodes:
        per_prim += ci.G * (4 + (3 if n.b0 is not None else 0) + 2)
    per_prim += ci.G * len(kv.targets)  # accumulate
    per_prim += 60
    once = 0
    hn, _ = build_hrr(ci.lc, ci.ld)
    once += ci.n_ebra * len(hn) * 2
    nk_c = ncart(ci.lc) * ncart(ci.ld)
    if spherical:
        td = sum(len(r) for r in transform_terms(ci.ld))
        tc = sum(len(r) for r in transform_terms(ci.lc))
        once += ci.n_ebra * (ncart(ci.lc) * td + nsph(ci.ld) * tc) * 2
    hb, _ = build_hrr(ci.la, ci.lb)
    once += ci.nket(spherical) * len(hb) * 2
    if spherical:
        tb = sum(len(r) for r in transform_terms(ci.lb))
        ta = sum(len(r) for r in transform_terms(ci.la))
        once += ci.nket(spherical) * (ncart(ci.la) * tb + nsph(ci.lb) * ta) * 2
    return per_prim * K4 + once, per_prim, once


def dag_flops(ci: ClassInfo, spherical: bool):
    """Algorithmic FP64 operations of the recurrence DAG this library evaluates.

    Counts each needed node once (FMA = 2 operations): the bra-phase nodes
    [e0|00]^(m) and ket-phase nodes [e0|f0]^(m) reachable from the targets
    (|e| in [la, la+lb], |f| in [lc, lc+ld], m = 0) under the chosen raise
    axes, the per-primitive-quartet geometry and Boys evaluation, the
    contraction adds, and the once-per-quartet horizontal recurrences and
    transforms.  Returns (per primitive quartet, per quartet).
    """
    Lb, Lk, L = ci.Lb, ci.Lk, ci.L
    kv = build_ket_vrr(ci.lc, Lk)
    knode = {(n.f, n.m): n for n in kv.nodes}
    need = set()
    stack = [(e, f, 0) for e in ci.lanes if sum(e) >= ci.la for (f, _) in kv.targets]
    flops = 0
    while stack:
        e, f, m = stack.pop()
        if (e, f, m) in need:
            continue
        need.add((e, f, m))
        if sum(f) > 0:
            n = knode[(f, m)]
            ax = n.axis
            flops += 3
            stack += [(e, n.a0[0], n.a0[1]), (e, n.a1[0], n.a1[1])]
            if n.b0 is not None:
                flops += 4
                stack += [(e, n.b0[0], n.b0[1]), (e, n.b1[0], n.b1[1])]
            if e[ax] > 0:
                flops += 2
                stack.append((sub(e, ax), n.a1[0], n.a1[1]))
        elif sum(e) > 0:
            # bra path built x, then y, then z: the last raise is along the last non-zero axis
            ax = 2 if e[2] > 0 else (1 if e[1] > 0 else 0)
            flops += 3
            e1 = sub(e, ax)
            stack += [(e1, f, m), (e1, f, m + 1)]
            if e[ax] >= 2:
                flops += 4
                e2 = sub(e, ax, 2)
                stack += [(e2, f, m), (e2, f, m + 1)]
    per_prim = flops
    per_prim += 30 + 14 + 3 * L + (L + 1)  # geometry and Boys
    per_prim += ci.n_ebra * len(kv.targets)  # contraction adds
    once = 0
    hn, _ = build_hrr(ci.lc, ci.ld)
    once += ci.n_ebra * len(hn) * 2
    if spherical:
        td = sum(len(r) for r in transform_terms(ci.ld))
        tc = sum(len(r) for r in transform_terms(ci.lc))
        once += ci.n_ebra * (ncart(ci.lc) * td + nsph(ci.ld) * tc) * 2
    hb, _ = build_hrr(ci.la, ci.lb)
    once += ci.nket(spherical) * len(hb) * 2
    if spherical:
        tb = sum(len(r) for r in transform_terms(ci.lb))
        ta = sum(len(r) for r in transform_terms(ci.la))
        once += ci.nket(spherical) * (ncart(ci.la) * tb + nsph(ci.lb) * ta) * 2
    return per_prim, once


# ---------------------------------------------------------------------------
# liveness-aware ordering of a lane's straight-line DAG ("FusionRCG" section
# III-A: the evaluation order of a fixed graph decides PeakLive, Eq. (4))
# ---------------------------------------------------------------------------

def peak_live(order, deps, initial=()):
    """PeakLive of a straight-line order: a value is live from its definition
    until its last consumer in the order (sinks define nothing)."""
    last = {}
    for t, (k, ds, sink) in enumerate(order):
        for d in ds:
            last[d] = t
    live = {k for k in initial if k in last}
    peak = len(live)
    for t, (k, ds, sink) in enumerate(order):
        if not sink and k in last:
            live.add(k)
        peak = max(peak, len(live))
        for d in ds:
            if last.get(d) == t:
                live.discard(d)
    return peak


def schedule_min_live(items, initial=(), remote=None, min_dist=0):
    """Greedy list scheduling that keeps few values live.

    items: [(key, deps, sink)] in any topological order.  At each step, among
    the ready items, pick the one that frees the most values net of the one it
    creates; ties go to the item whose value is needed soonest by a ready-ish
    consumer (most recently readied operand chain), then to the original order.
    This plays the role of the page's DSA heuristic (Eq. (7)) on our graphs.

    remote: optional {key: source key} of a cross-lane operand; such an item is
    deferred (while anything else is ready) until its source was produced at
    least ``min_dist`` steps earlier, so the cross-lane read can be issued that
    far ahead of its use.
    """
    from . import variant
    if variant.CURRENT.schedule == "topo":
        return topo_order(items)
    remote = remote or {}
    n = len(items)
    idx_of = {k: i for i, (k, ds, s) in enumerate(items)}
    uses = {}
    consumers = {}
    for i, (k, ds, s) in enumerate(items):
        for d in ds:
            uses[d] = uses.get(d, 0) + 1
            consumers.setdefault(d, []).append(i)
    avail = set(initial)
    missing = [sum(1 for d in ds if d in idx_of) for (k, ds, s) in items]
    ready = {i for i in range(n) if missing[i] == 0}
    done = [False] * n
    order = []
    stamp = {i: 0 for i in ready}
    clock = 0
    born = {}
    while ready:
        best, bscore = None, None
        for i in ready:
            k, ds, s = items[i]
            freed = sum(1 for d in set(ds) if uses.get(d, 0) == ds.count(d) and d not in ())
            rs = remote.get(k)
            early = rs is not None and rs in born and clock - born[rs] < min_dist
            score = (not early, freed - (0 if s else 1), stamp[i], -i)
            if bscore is None or score > bscore:
                best, bscore = i, score
        ready.remove(best)
        done[best] = True
        k, ds, s = items[best]
        order.append(items[best])
        born[k] = clock
        for d in ds:
            uses[d] -= 1
        clock += 1
        for c in consumers.get(k, []):
            missing[c] -= 1
            if missing[c] == 0:
                ready.add(c)
                stamp[c] = clock
    assert len(order) == n, "cycle or missing dependency"
    return order


def topo_order(items):
    """A plain topological order of the same items: Kahn's algorithm taking the
    ready item that comes first in the given order (no liveness objective; the
    plain valid ordering without liveness optimisation that section V-B of
    "FusionRCG" compares DSA against)."""
    import heapq
    n = len(items)
    idx_of = {k: i for i, (k, ds, s) in enumerate(items)}
    consumers = {}
    missing = [0] * n
    for i, (k, ds, s) in enumerate(items):
        for d in ds:
            if d in idx_of:
                missing[i] += 1
                consumers.setdefault(d, []).append(i)
    heap = [i for i in range(n) if missing[i] == 0]
    heapq.heapify(heap)
    order = []
    while heap:
        i = heapq.heappop(heap)
        order.append(items[i])
        for c in consumers.get(items[i][0], []):
            missing[c] -= 1
            if missing[c] == 0:
                heapq.heappush(heap, c)
    assert len(order) == n, "cycle or missing dependency"
    return order
