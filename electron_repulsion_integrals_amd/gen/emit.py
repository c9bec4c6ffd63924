"""Emit one HIP source per angular-momentum class (register tier and memory tier).

Both tiers share the algorithm of graph.py; they differ in where values live:

* register tier ("V"): the whole quartet lives in VGPRs of a lane group of
  G = #{e : |e| <= la+lb} lanes inside one wave64; floor(64/G) quartets per
  wave.  The coupling operand is read from lane e-1_i with ds_bpermute.  The
  ket results are handed from "lane owns e" to "lane owns ket component"
  through one LDS transpose per quartet.
* memory tier ("M"): for classes whose lane group exceeds a wave or whose live
  set exceeds the register budget.  One workgroup per quartet, lane = e; every
  graph value lives in a per-workgroup slice of a global scratch buffer,
  interleaved so that lanes of a wave touch consecutive doubles.  Slots are
  reused once a value is dead (two-pass lifetime allocation, as the page's
  Tier 2 kernel does with its global buffer), and workgroup barriers separate
  the ket levels because the coupling operand may belong to another wave.
"""
from __future__ import annotations

import os

from .cartesian import components, components_upto, sub, add, ncart, nsph, comp_index
from .graph import (ClassInfo, build_ket_vrr, build_hrr, transform_terms, class_id, ket_vrr_peak_live)

AX = "xyz"

# cross-lane reads are issued this many ops ahead of their use, and pinned there:
# a scheduling barrier that only ALU work may cross keeps the compiler from
# sinking them back next to their consumers (their LDS latency then overlaps
# the arithmetic in between)
REMOTE_AHEAD = 6
PIN_REMOTE = True
# a node reading a neighbour's value is scheduled at least this many ops after
# that value is produced (when anything else is ready)
REMOTE_DIST = 10


def _fmt(v: float) -> str:
    r = repr(float(v))
    if "e" not in r and "." not in r and "inf" not in r and "nan" not in r:
        r += ".0"
    return r


# ---------------------------------------------------------------------------
# value naming helpers
# ---------------------------------------------------------------------------

class Names:
    """Maps graph values to C expressions for a given storage tier."""

    def __init__(self, tier, kv, Lk, slot_of=None):
        self.tier = tier
        self.fpos = {f: i for i, f in enumerate(components_upto(max(Lk, 0)))}
        self.slot_of = slot_of or {}

    def ket(self, node):
        f, m = node
        if sum(f) == 0:
            return f"s1_{m}"
        if self.tier == "V":
            return f"v{self.fpos[f]}_{m}"
        return f"SLD({self.slot_of[('k', f, m)]})"

    def ket_store(self, node, expr):
        f, m = node
        return f"SST({self.slot_of[('k', f, m)]}, {expr})"

    def ket_remote(self, node, axis):
        f, m = node
        if self.tier == "V":
            return f"eri_bperm(ad{AX[axis]}, {self.ket(node)})"
        if sum(f) == 0:
            raise AssertionError("remote base values are read from the remote lane's own stage-1 copy")
        return f"SLDL({self.slot_of[('k', f, m)]}, src{AX[axis]})"


# ---------------------------------------------------------------------------
# slot allocation for the memory tier
# ---------------------------------------------------------------------------

def _alloc_slots(kv):
    """Level-granular lifetime packing of the ket-phase values.

    A value produced at level k is read at levels k+1 (own and coupling) and
    k+2 (the f-2_i term).  Slots are released only at level boundaries so that
    the barrier between levels also orders every read before any reuse.
    """
    level_of = {}
    last_level = {}
    for n in kv.nodes:
        k = sum(n.f)
        level_of[(n.f, n.m)] = k
        for p in (n.a0, n.a1, n.b0, n.b1):
            if p is not None and sum(p[0]) > 0:
                last_level[p] = max(last_level.get(p, 0), k)
    # targets are accumulated at the level they are produced
    for t in kv.targets:
        if sum(t[0]) > 0:
            last_level[t] = max(last_level.get(t, 0), level_of[t])
    slot_of = {}
    free = []
    nslots = 0
    by_level = {}
    for n in kv.nodes:
        by_level.setdefault(sum(n.f), []).append((n.f, n.m))
    release_at = {}
    for v, lv in last_level.items():
        release_at.setdefault(lv, []).append(v)
    for k in sorted(by_level):
        for v in by_level[k]:
            if free:
                s = free.pop()
            else:
                s = nslots
                nslots += 1
            slot_of[("k",) + v] = s
        # values whose last use is at level k free their slot for level k+1
        for v in release_at.get(k, []):
            free.append(slot_of[("k",) + v])
        free.sort(reverse=True)
    return slot_of, nslots


# ---------------------------------------------------------------------------
# code pieces
# ---------------------------------------------------------------------------

def _stage1_selectors(ci: ClassInfo, lines, stride, one_field, zero_field, ind="  ", compact=None):
    """Per-lane record offsets of the bra-path factors: step s of lane e moves
    along axis ax_s, so it needs (P-A)_ax (record field ax) and (W-P)_ax (field
    3 + ax); a lane whose path is shorter than the step reads the constant
    fields 1 and 0, which leave its values unchanged.  Loop-invariant ints:
    each step then costs two LDS reads instead of selects among six doubles.
    compact="all": the two offsets and the step's lowering count n (bits 0-11,
    12-23 and 24-26) share one int per step, unpacked inside the primitive loop:
    one register per step instead of four across the loop."""
    for s in range(1, ci.Lb + 1):
        lines.append(f"{ind}const int ax{s} = ({s} <= ex) ? 0 : ({s} <= ex + ey) ? 1 : ({s} <= es) ? 2 : 3;")
        sel1 = f"(ax{s} < 3 ? ax{s} : {one_field}) * {stride}"
        sel2 = f"(ax{s} < 3 ? 3 + ax{s} : {zero_field}) * {stride}"
        gnf = f"(ax{s} == 0 ? {s - 1} : ax{s} == 1 ? {s - 1} - ex : ax{s} == 2 ? {s - 1} - ex - ey : 0)"
        if compact == "all":
            if s == 1:
                lines.append(f"{ind}static_assert(({one_field} + 1) * {stride} <= 4096 && "
                             f"({zero_field} + 1) * {stride} <= 4096 && {ci.Lb} <= 8, \"selector fields\");")
            lines.append(f"{ind}const int selp{s} = ({sel1}) | (({sel2}) << 12) | ({gnf} << 24);")
            continue
        lines.append(f"{ind}const int sel1_{s} = {sel1};")
        lines.append(f"{ind}const int sel2_{s} = {sel2};")
        lines.append(f"{ind}const double gnf{s} = (double){gnf};")


STEP1_SHORTCUT = True


def _stage1(ci: ClassInfo, base_m: int, lines, ind="      ", rsel=None, compact=None, shortcut=None):
    """Bra phase for the lane's own e: [e0|00]^(m), m = 0..base_m, from F_m.
    rsel: name of this lane's record pointer (factors read through the
    selectors of _stage1_selectors, packed ones with compact); otherwise
    selects on PAx.. WPz.  shortcut (default STEP1_SHORTCUT) drops the lowering
    term of the first step, which is zero there."""
    if shortcut is None:
        shortcut = STEP1_SHORTCUT
    L = ci.L
    for m in range(L + 1):
        lines.append(f"{ind}double c{m} = F[{m}];")
    if ci.Lb == 0:
        for m in range(base_m + 1):
            lines.append(f"{ind}const double s1_{m} = c{m};")
        return
    for m in range(L + 1):
        lines.append(f"{ind}double p{m} = 0.0;")
    for s in range(1, ci.Lb + 1):
        top = L - s
        lines.append(f"{ind}{{ // bra step {s}")
        if rsel is not None and compact == "all":
            # the empty asm makes the packed selector opaque in the loop, so that
            # its unpacked fields are not hoisted out as loop invariants again
            lines.append(f"{ind}  int sp = selp{s};")
            lines.append(f'{ind}  asm volatile("" : "+v"(sp));')
            lines.append(f"{ind}  const double g1 = {rsel}[sp & 4095], g2 = {rsel}[(sp >> 12) & 4095];")
            lines.append(f"{ind}  const double gn = (double)(sp >> 24) * i2z;")
        elif rsel is not None:
            lines.append(f"{ind}  const double g1 = {rsel}[sel1_{s}], g2 = {rsel}[sel2_{s}];")
            lines.append(f"{ind}  const double gn = gnf{s} * i2z;")
        else:
            lines.append(f"{ind}  const int ax = ({s} <= ex) ? 0 : ({s} <= ex + ey) ? 1 : ({s} <= es) ? 2 : 3;")
            lines.append(f"{ind}  const double g1 = ax == 0 ? PAx : ax == 1 ? PAy : ax == 2 ? PAz : 1.0;")
            lines.append(f"{ind}  const double g2 = ax == 0 ? WPx : ax == 1 ? WPy : ax == 2 ? WPz : 0.0;")
            lines.append(f"{ind}  const double gn = (double)(ax == 0 ? {s - 1} : ax == 1 ? {s - 1} - ex : "
                         f"ax == 2 ? {s - 1} - ex - ey : 0) * i2z;")
        for m in range(top + 1):
            if s == 1 and shortcut:  # nothing to lower yet: the p terms are zero
                lines.append(f"{ind}  const double n{m} = g1 * c{m} + g2 * c{m + 1};")
            else:
                lines.append(f"{ind}  const double n{m} = g1 * c{m} + g2 * c{m + 1} + gn * (p{m} - roz * p{m + 1});")
        if s == 1 and shortcut:
            lines.append(f"{ind}  (void)gn;")
        for m in range(top + 1):
            lines.append(f"{ind}  p{m} = c{m}; c{m} = n{m};")
        lines.append(f"{ind}}}")
    for m in range(base_m + 1):
        lines.append(f"{ind}const double s1_{m} = c{m};")


def _ket_phase(kv, names: Names, lines, ind="      ", barrier=None, acc_now=None):
    """Ket phase of Eq. (2) in node order.  ``acc_now`` maps a target node to
    the accumulator it is added to immediately (memory tier: before its slot
    can be reused at a later level)."""
    prev_level = None
    remote_name = {}
    nodes = kv.nodes
    defined = set()

    def issue_remote(j):
        # a cross-lane read may be issued once its source (previous level) exists
        m2 = nodes[j]
        key = (m2.a1, m2.axis)
        if key in remote_name:
            return
        if sum(m2.a1[0]) > 0 and m2.a1 not in defined:
            return
        remote_name[key] = f"xr{len(remote_name)}"
        lines.append(f"{ind}const double {remote_name[key]} = {names.ket_remote(m2.a1, m2.axis)};")

    for idx, n in enumerate(nodes):
        lvl = sum(n.f)
        if barrier and prev_level is not None and lvl != prev_level:
            lines.append(f"{ind}{barrier}")
        if names.tier == "V":
            # sliding window: issue the reads of the next REMOTE_AHEAD nodes now so
            # that their LDS latency overlaps the arithmetic in between
            for j in range(idx, min(len(nodes), idx + REMOTE_AHEAD + 1)):
                issue_remote(j)
            issue_remote(idx)
        prev_level = lvl
        a = AX[n.axis]
        expr = f"QC{a} * {names.ket(n.a0)} + WQ{a} * {names.ket(n.a1)}"
        if n.b0 is not None:
            expr += f" + {_fmt(n.fi_minus_1)} * i2e * ({names.ket(n.b0)} - roe * {names.ket(n.b1)})"
        if names.tier == "V":
            expr += f" + eh{a} * {remote_name[(n.a1, n.axis)]}"
        elif sum(n.a1[0]) > 0:
            expr += f" + eh{a} * {names.ket_remote(n.a1, n.axis)}"
        else:
            # memory tier, coupling to the remote lane's bra-phase value
            expr += f" + eh{a} * S1L({n.a1[1]}, src{a})"
        if names.tier == "V":
            lines.append(f"{ind}const double {names.ket((n.f, n.m))} = {expr};")
            defined.add((n.f, n.m))
        else:
            lines.append(f"{ind}{{ const double t_ = {expr}; {names.ket_store((n.f, n.m), 't_')};")
            if acc_now is not None and (n.f, n.m) in acc_now:
                a = acc_now[(n.f, n.m)]
                lines.append(f"{ind}  SST({a}, SLD({a}) + t_);")
            lines.append(f"{ind}}}")


def _hrr_block(l1, l2, base_expr, R, out_prefix, spherical, lines, ind="  ", decl="double"):
    """HRR (x, y) from base (e, 0) then optional transform of y then x.

    base_expr(e) -> C expression of the base value (e, 0).  R is the name prefix
    of the centre difference (ABx.. or CDx..).  Emits variables
    {out_prefix}{k} for output index k (row-major x, y; spherical or Cartesian).
    Returns the number of outputs.
    """
    nodes, base = build_hrr(l1, l2)
    name = {}
    for e in base:
        name[(e, (0, 0, 0))] = base_expr(e)
    for i, n in enumerate(nodes):
        nm = f"{out_prefix}h{i}"
        hi, lo = name[n.p_hi], name[n.p_lo]
        lines.append(f"{ind}const double {nm} = {hi} + {R}{AX[n.axis]} * {lo};")
        name[(n.x, n.y)] = nm
    xs, ys = components(l1), components(l2)
    outs = []
    if not spherical:
        for x in xs:
            for y in ys:
                outs.append(name[(x, y)])
    elif max(l1, l2) <= 2:
        # both indices at once: out = sum over non-zeros of t(l1) x t(l2)
        Ty, Tx = transform_terms(l2), transform_terms(l1)
        for li, rowx in enumerate(Tx):
            for si, rowy in enumerate(Ty):
                terms = [f"{_fmt(cx * cy)} * {name[(xs[xi], ys[yi])]}" for xi, cx in rowx for yi, cy in rowy]
                nm = f"{out_prefix}u{li}_{si}"
                lines.append(f"{ind}const double {nm} = {' + '.join(terms)};")
                outs.append(nm)
    else:
        Ty, Tx = transform_terms(l2), transform_terms(l1)
        # y first
        mid = {}
        for xi, x in enumerate(xs):
            for si, row in enumerate(Ty):
                terms = [f"{_fmt(c)} * {name[(x, ys[yi])]}" for yi, c in row]
                nm = f"{out_prefix}t{xi}_{si}"
                lines.append(f"{ind}const double {nm} = {' + '.join(terms)};")
                mid[(xi, si)] = nm
        for li, row in enumerate(Tx):
            for si in range(nsph(l2)):
                terms = [f"{_fmt(c)} * {mid[(xi, si)]}" for xi, c in row]
                nm = f"{out_prefix}u{li}_{si}"
                lines.append(f"{ind}const double {nm} = {' + '.join(terms)};")
                outs.append(nm)
    for k, nm in enumerate(outs):
        lines.append(f"{ind}{decl} {out_prefix}{k} = {nm};")
    return len(outs)


def _hrr_ops(l1, l2, R, spherical):
    """HRR (Eq. (3)) then transform of y then x, as a list of linear ops.

    Returns (ops, base, outputs): ops = [(key, [(coef, src_key)])] in order,
    coef a C expression or None for 1; base = list of base triples e (key
    ('b', e)); outputs = keys of the final values in output order.
    """
    nodes, base = build_hrr(l1, l2)
    key = {}
    for e in base:
        key[(e, (0, 0, 0))] = ("b", e)
    ops = []
    for n in nodes:
        k = ("h", n.x, n.y)
        ops.append((k, [(None, key[n.p_hi]), (f"{R}{AX[n.axis]}", key[n.p_lo])]))
        key[(n.x, n.y)] = k
    xs, ys = components(l1), components(l2)
    outs = []
    if not spherical:
        outs = [key[(x, y)] for x in xs for y in ys]
    else:
        Ty, Tx = transform_terms(l2), transform_terms(l1)
        # a Cartesian component x that only one spherical row of the first index
        # uses, with a single coefficient c: c is folded into the second index's
        # coefficients of the values t(x, .), and that row is t itself
        uses = {}
        for li, row in enumerate(Tx):
            for xi, c in row:
                uses.setdefault(xi, []).append(li)
        fold = {}
        for li, row in enumerate(Tx):
            if len(row) == 1 and len(uses[row[0][0]]) == 1:
                fold[row[0][0]] = row[0][1]
        for xi, x in enumerate(xs):
            f = fold.get(xi, 1.0)
            for si, row in enumerate(Ty):
                ops.append((("t", xi, si), [(_fmt(f * c), key[(x, ys[yi])]) for yi, c in row]))
        for li, row in enumerate(Tx):
            for si in range(nsph(l2)):
                k = ("u", li, si)
                if len(row) == 1 and row[0][0] in fold:
                    ops.append((k, [(None, ("t", row[0][0], si))]))
                else:
                    ops.append((k, [(_fmt(c), ("t", xi, si)) for xi, c in row]))
                outs.append(k)
    return ops, base, outs


def _emit_ops_mem(ops, base_expr, outs, store, slot_base, lines, ind):
    """Emit ops with every intermediate in a private scratch slot (linear-scan reuse).

    base_expr(e) reads a base value; store(k, expr) emits the statement that
    consumes output k.  Returns the number of private slots used.
    """
    last = {}
    for t, (k, terms) in enumerate(ops):
        for _, src in terms:
            last[src] = t
    out_set = set(outs)
    free, nslot, slot = [], 0, {}

    def ref(src):
        if src[0] == "b":
            return base_expr(src[1])
        return f"SLD({slot_base + slot[src]})"

    for t, (k, terms) in enumerate(ops):
        parts = []
        for coef, src in terms:
            parts.append(ref(src) if coef is None else f"{coef} * {ref(src)}")
        expr = " + ".join(parts)
        # release sources whose last use is this op before allocating the result
        for _, src in terms:
            if src[0] != "b" and last.get(src) == t and src not in out_set and src in slot:
                free.append(slot.pop(src))
        if k in out_set and k not in last:
            lines.append(f"{ind}{store(outs.index(k), expr)}")
            continue
        if free:
            sidx = free.pop()
        else:
            sidx = nslot
            nslot += 1
        slot[k] = sidx
        lines.append(f"{ind}SST({slot_base + sidx}, {expr});")
    # outputs that are also intermediates (Cartesian) are stored after the sweep;
    # with a zero second angular momentum the outputs are the base values themselves
    for i, k in enumerate(outs):
        if k in slot:
            lines.append(f"{ind}{store(i, f'SLD({slot_base + slot[k]})')}")
        elif k[0] == "b":
            lines.append(f"{ind}{store(i, base_expr(k[1]))}")
    return nslot


# ---------------------------------------------------------------------------
# register tier
# ---------------------------------------------------------------------------

def emit_register_tier(ci: ClassInfo, spherical: bool) -> str:
    """Two kernels per class: general (contracted) and K4 = 1 (no accumulators).

    Both run a persistent grid-stride loop over groups of Q quartets and load the
    next group's indices, pair records and centres while the current group
    computes, so the dependent load chain of a quartet is hidden.
    """
    from .lane import use_lane_tier
    lane_tier = USE_LANE_TIER and use_lane_tier(ci, spherical)
    layout = ("lane tier: one quartet per lane" if lane_tier else
              f"register tier: {ci.G} lanes per quartet, {64 // ci.G} quartets per wave")
    out = [f"// class ({ci.la}{ci.lb}|{ci.lc}{ci.ld}) id {class_id(ci.la, ci.lb, ci.lc, ci.ld)}, "
           f"{'spherical' if spherical else 'Cartesian'} output, {layout}",
           '#include "eri_device.h"', ""]
    from .packed import use_packed_k1, emit_packed_k1, use_packed_contracted, emit_packed_contracted
    from .lane import emit_lane_tier
    if lane_tier:
        out += emit_lane_tier(ci, spherical, False)
        out += emit_lane_tier(ci, spherical, True)
        return "\n".join(out) + "\n"
    # a lane group wider than a wave exists only as a packed multi-wave workgroup
    assert ci.G <= 64 or (use_packed_contracted(ci, spherical) and use_packed_k1(ci, spherical)), ci
    if use_packed_contracted(ci, spherical):
        out += emit_packed_contracted(ci, spherical)
    else:
        out += _register_kernel(ci, spherical, k1=False)
    batched = BATCH_K1 and ci.G >= K1_BATCH_MIN_G
    if use_packed_k1(ci, spherical):
        out += emit_packed_k1(ci, spherical)
    elif batched:
        out += _register_kernel_k1_batched(ci, spherical)
    else:
        out += _register_kernel(ci, spherical, k1=True)
    return "\n".join(out) + "\n"


BATCH_K1 = True
USE_LANE_TIER = True
SELECT_LDS_CONTRACTED = True
K1_BATCH = 32  # quartet records set up together, one per lane
K1_BATCH_MIN_G = 8  # narrower lane groups repeat the set-up in few lanes: per-group set-up


def _register_kernel_k1_batched(ci: ClassInfo, spherical: bool):
    """K4 = 1 kernel with batched set-up.  A wave walks its groups g, g + grid,
    g + 2 grid, ...; every RB groups, each of the first RB x Q lanes computes
    the geometry and Boys values of one quartet of the next RB groups into an
    LDS record (field-major).  The serial set-up chain (pair records, exp,
    reciprocals, square root, Boys table) then runs once per batch in parallel
    lanes instead of once per quartet in all lanes."""
    kv = build_ket_vrr(ci.lc, ci.Lk)
    names = Names("V", kv, ci.Lk)
    G = ci.G
    Q = 64 // G
    RB = max(1, K1_BATCH // Q)
    NK = ci.nket(spherical)
    NEB = ci.n_ebra
    EOFF = ci.e_bra_offset
    BLK = ci.nout(spherical)
    L = ci.L
    cid = class_id(ci.la, ci.lb, ci.lc, ci.ld)
    tag = f"c{cid}_{'s' if spherical else 'c'}_k1"
    lanes = ci.lanes
    lpos = {e: i for i, e in enumerate(lanes)}
    lane_tab = []
    for e in lanes:
        d = [lpos[sub(e, ax)] if e[ax] > 0 else -1 for ax in range(3)]
        lane_tab.append(e[0] | (e[1] << 4) | (e[2] << 8) | ((d[0] + 1) << 12) | ((d[1] + 1) << 18) | ((d[2] + 1) << 24))
    fields = REC_FIELDS + [f"F{m}" for m in range(L + 1)] + ["CDx", "CDy", "CDz", "ABx", "ABy", "ABz"]
    NR = len(fields) + 2  # then two constant rows, 1.0 and 0.0, for the bra-path selectors
    NRL = RB * Q  # records per batch
    o = []
    o.append("namespace {")
    o.append(f"__constant__ int k_{tag}_lane[{G}] = {{" + ", ".join(str(v) for v in lane_tab) + "};")
    o.append("}  // namespace")
    o.append(f"__global__ void __launch_bounds__(64) eri_kernel_{tag}(EriClassArgs a)")
    o.append("{")
    o.append(f"  constexpr int G = {G}, Q = {Q}, NK = {NK}, NEB = {NEB}, BLK = {BLK}, RB = {RB}, NRL = {NRL};")
    # field stride of the records: odd, so that lanes reading different fields of
    # one record (the bra-path selectors) hit different LDS banks
    o.append(f"  constexpr int RS = {NRL | 1};")
    o.append("  __shared__ double xch[Q * NEB * NK + NK];  // exchange rows, then a junk row")
    o.append(f"  __shared__ double rec[{NR} * RS];  // field-major quartet records of one batch")
    o.append("  const int lane = threadIdx.x;")
    o.append("  int grp = lane / G, sub = lane - grp * G;")
    o.append("  if (grp >= Q) { grp = Q; sub = 0; }  // padding lanes: phantom group, e = (0,0,0)")
    o.append(f"  const int lt = k_{tag}_lane[sub];")
    o.append("  const int ex = lt & 15, ey = (lt >> 4) & 15, ez = (lt >> 8) & 15, es = ex + ey + ez;")
    o.append("  const int gb = grp * G;")
    o.append("  const int adx = (ex > 0 ? gb + ((lt >> 12) & 63) - 1 : lane) * 4;")
    o.append("  const int ady = (ey > 0 ? gb + ((lt >> 18) & 63) - 1 : lane) * 4;")
    o.append("  const int adz = (ez > 0 ? gb + ((lt >> 24) & 63) - 1 : lane) * 4;")
    o.append("  (void)adx; (void)ady; (void)adz; (void)es;")
    o.append("  const int ngroups = (a.nq + Q - 1) / Q;")
    o.append("  const int rq = grp < Q ? grp : 0;  // record member of this lane's group")
    o.append(f"  if (lane < NRL) {{ rec[{NR - 2} * RS + lane] = 1.0; rec[{NR - 1} * RS + lane] = 0.0; }}")
    _stage1_selectors(ci, o, "RS", NR - 2, NR - 1)
    o.append("  int it = 0;")
    o.append("  for (int g = blockIdx.x; g < ngroups; g += (int)gridDim.x, ++it) {")
    o.append("    const int bslot = it % RB;")
    o.append("    if (bslot == 0) {")
    o.append("      if (lane < NRL) {")
    o.append("        const int k = lane / Q, gk = g + k * (int)gridDim.x;")
    o.append("        int q = gk * Q + (lane - k * Q);")
    o.append("        if (gk >= ngroups || q >= a.nq) q = a.nq - 1;  // past the end: a valid record, never used")
    # explicit lists are the identity pairing: one dependent load less
    o.append("        const int bra = a.pair_base >= 0 ? (int)(a.pair_base + 2 * (long long)q) : a.qbra[q];")
    o.append("        const int ket = a.pair_base >= 0 ? bra + 1 : a.qket[q];")
    o.append("        const int4 pb = a.pair_info[bra], pk = a.pair_info[ket];")
    o.append("        const double Ax = a.cen[3 * pb.x], Ay = a.cen[3 * pb.x + 1], Az = a.cen[3 * pb.x + 2];")
    o.append("        const double Cx = a.cen[3 * pk.x], Cy = a.cen[3 * pk.x + 1], Cz = a.cen[3 * pk.x + 2];")
    o.append("        const EriPrimPair P = eri_load_pp(a.ppd, pb.z);")
    o.append("        const EriPrimPair K = eri_load_pp(a.ppd, pk.z);")
    o.append("        EriQuartetGeom gq;")
    o.append("        eri_geom(P, K, Ax - Cx, Ay - Cy, Az - Cz, gq);")
    o.append(f"        double F[{L + 1}];")
    o.append(f"        eri_boys<{L}>(gq.T, gq.pref, a.boys, F);")
    vals = ["P.PA[0]", "P.PA[1]", "P.PA[2]", "gq.WP[0]", "gq.WP[1]", "gq.WP[2]", "K.PA[0]", "K.PA[1]", "K.PA[2]",
            "gq.WQ[0]", "gq.WQ[1]", "gq.WQ[2]", "0.5 * P.izeta", "0.5 * K.izeta", "gq.roz", "gq.roe", "gq.i2ze"]
    vals += [f"F[{m}]" for m in range(L + 1)]
    vals += ["Cx - a.cen[3 * pk.y]", "Cy - a.cen[3 * pk.y + 1]", "Cz - a.cen[3 * pk.y + 2]",
             "Ax - a.cen[3 * pb.y]", "Ay - a.cen[3 * pb.y + 1]", "Az - a.cen[3 * pb.y + 2]"]
    assert len(vals) == NR - 2
    o.append("        double* r = rec + lane;")
    for fi, v in enumerate(vals):
        o.append(f"        r[{fi} * RS] = {v};")
    o.append("      }")
    o.append("      __syncthreads();")
    o.append("    }")
    o.append("    {")
    o.append("      const double* r = rec + bslot * Q + rq;")
    for fi, nm in enumerate(fields):
        if nm.startswith("F") or fi < 6:  # P-A and W-P are read by the bra path through its selectors
            continue
        o.append(f"      const double {nm} = r[{fi} * RS];")
    o.append(f"      double F[{L + 1}];")
    for m in range(L + 1):
        o.append(f"      F[{m}] = r[{len(REC_FIELDS) + m} * RS];")
    o.append("      (void)CDx; (void)CDy; (void)CDz; (void)ABx; (void)ABy; (void)ABz;")
    o.append("      const double ehx = ex * i2ze, ehy = ey * i2ze, ehz = ez * i2ze;")
    o.append("      (void)QCx; (void)QCy; (void)QCz;")
    o.append("      (void)WQx; (void)WQy; (void)WQz; (void)i2z; (void)i2e; (void)roz; (void)roe; (void)ehx; (void)ehy; (void)ehz;")
    _stage1(ci, kv.base_m, o, "      ", rsel="r")
    o.append(f"      double* xd = xch + ((grp < Q && es >= {ci.la}) ? (grp * NEB + (sub - {EOFF})) * NK : Q * NEB * NK);")
    init_keys = [("k", (0, 0, 0), m) for m in range(kv.base_m + 1)]
    _emit_scheduled(_lane_ops(ci, kv, names, spherical, True), init_keys, names, o, "      ")
    o.append("    }")
    o.append("    __syncthreads();")
    # H2: lanes own ket components
    o.append("    for (int t = lane; t < Q * NK; t += 64) {")
    o.append("      const int g2 = t / NK, kap = t - g2 * NK;")
    o.append("      const int slot = g * Q + g2;")
    o.append("      if (slot >= a.nq) continue;")
    ab0 = fields.index("ABx")
    o.append(f"      const double* r = rec + bslot * Q + g2;")
    o.append(f"      const double ABx = r[{ab0} * RS], ABy = r[{ab0 + 1} * RS], ABz = r[{ab0 + 2} * RS];")
    o.append("      (void)ABx; (void)ABy; (void)ABz;")
    o.append("      const double* src = xch + g2 * NEB * NK + kap;")
    ebra = [e for l in range(ci.la, ci.Lb + 1) for e in components(l)]
    epos = {e: i for i, e in enumerate(ebra)}
    o.append("      double* dst = a.out + (size_t)slot * BLK + kap;")
    _emit_hrr_scheduled(ci.la, ci.lb, lambda e: f"src[{epos[e]} * NK]", "AB", spherical,
                        lambda k, x: f"eri_out(&dst[{k} * NK], {x});", o, "      ", "z")
    o.append("    }")
    o.append("    __syncthreads();  // exchange and records are rewritten next")
    o.append("  }")
    o.append("}")
    o.append("")
    o.append(f"void eri_launch_{tag}(const EriClassArgs& a, hipStream_t s)")
    o.append("{")
    o.append(f"  const int ngroups = (a.nq + {Q} - 1) / {Q};")
    o.append("  const int nblk = ngroups < a.grid_cap ? ngroups : a.grid_cap;")
    o.append(f"  if (nblk > 0) hipLaunchKernelGGL(eri_kernel_{tag}, dim3(nblk), dim3(64), 0, s, a);")
    o.append("}")
    o.append("")
    return o




# ---------------------------------------------------------------------------
# liveness-ordered emission of a lane's straight-line graph (register tier)
# ---------------------------------------------------------------------------

def _lane_ops(ci, kv, names, spherical, k1, store_prefix="xd"):
    """Ops of one lane as (key, deps, sink, emit(remote_name) -> C lines).

    k1: ket recurrence -> ket HRR -> ket transform -> exchange stores.
    otherwise: ket recurrence -> accumulator adds (inside the primitive loop).
    """
    ops = []
    for n in kv.nodes:
        ds = [("k",) + n.a0, ("k",) + n.a1] + ([("k",) + n.b0, ("k",) + n.b1] if n.b0 else [])

        def emit(rn, n=n):
            a = AX[n.axis]
            expr = f"QC{a} * {names.ket(n.a0)} + WQ{a} * {names.ket(n.a1)}"
            if n.b0 is not None:
                expr += f" + {_fmt(n.fi_minus_1)} * i2e * ({names.ket(n.b0)} - roe * {names.ket(n.b1)})"
            expr += f" + eh{a} * {rn}"
            return [f"const double {names.ket((n.f, n.m))} = {expr};"]
        ops.append((("k", n.f, n.m), ds, False, emit, (n.a1, n.axis)))
    if not k1:
        for t, tg in enumerate(kv.targets):
            src = ("k",) + tg
            ops.append((("acc", t), [src] if sum(tg[0]) > 0 else [], True,
                        (lambda rn, t=t, tg=tg: [f"acc{t} += {names.ket(tg)};"]), None))
        return ops
    hn, base = build_hrr(ci.lc, ci.ld)
    key = {(e, (0, 0, 0)): ("k", e, 0) for e in base}
    cname = {}

    def nm(k):
        if k[0] == "k":
            return names.ket((k[1], k[2]))
        return cname[k]
    for i, n in enumerate(hn):
        k = ("h", n.x, n.y)
        cname[k] = f"yh{i}"
        hi, lo = key[n.p_hi], key[n.p_lo]
        ops.append((k, [hi, lo], False,
                    (lambda rn, k=k, hi=hi, lo=lo, ax=n.axis: [f"const double {cname[k]} = {nm(hi)} + CD{AX[ax]} * {nm(lo)};"]),
                    None))
        key[(n.x, n.y)] = k
    xs, ys = components(ci.lc), components(ci.ld)
    outs = []
    if not spherical:
        outs = [key[(x, y)] for x in xs for y in ys]
    elif max(ci.lc, ci.ld) <= 2:
        Ty, Tx = transform_terms(ci.ld), transform_terms(ci.lc)
        for li, rowx in enumerate(Tx):
            for si, rowy in enumerate(Ty):
                k = ("u", li, si)
                cname[k] = f"yu{li}_{si}"
                terms = [(cx * cy, key[(xs[xi], ys[yi])]) for xi, cx in rowx for yi, cy in rowy]
                ops.append((k, [t for _, t in terms], False,
                            (lambda rn, k=k, terms=terms: [f"const double {cname[k]} = " +
                                                          " + ".join(f"{_fmt(c)} * {nm(t)}" for c, t in terms) + ";"]),
                            None))
                outs.append(k)
    else:
        Ty, Tx = transform_terms(ci.ld), transform_terms(ci.lc)
        for xi, x in enumerate(xs):
            for si, row in enumerate(Ty):
                k = ("t", xi, si)
                cname[k] = f"yt{xi}_{si}"
                terms = [(c, key[(x, ys[yi])]) for yi, c in row]
                ops.append((k, [t for _, t in terms], False,
                            (lambda rn, k=k, terms=terms: [f"const double {cname[k]} = " +
                                                          " + ".join(f"{_fmt(c)} * {nm(t)}" for c, t in terms) + ";"]),
                            None))
        for li, row in enumerate(Tx):
            for si in range(nsph(ci.ld)):
                k = ("u", li, si)
                cname[k] = f"yu{li}_{si}"
                terms = [(c, ("t", xi, si)) for xi, c in row]
                ops.append((k, [t for _, t in terms], False,
                            (lambda rn, k=k, terms=terms: [f"const double {cname[k]} = " +
                                                          " + ".join(f"{_fmt(c)} * {nm(t)}" for c, t in terms) + ";"]),
                            None))
                outs.append(k)
    for i, ok in enumerate(outs):
        ops.append((("w", i), [ok], True, (lambda rn, i=i, ok=ok: [f"{store_prefix}[{i}] = {nm(ok)};"]), None))
    return ops


def _emit_scheduled(ops, initial, names, lines, ind, ahead=None):
    """Order ops by schedule_min_live, issue cross-lane reads `ahead` ops early."""
    from .graph import schedule_min_live
    if ahead is None:
        ahead = REMOTE_AHEAD
    items = [(k, ds, sink) for (k, ds, sink, _, _) in ops]
    remote = {k: ("k",) + rem[0] for (k, ds, sink, _, rem) in ops if rem is not None and sum(rem[0][0]) > 0}
    order = schedule_min_live(items, initial, remote, REMOTE_DIST)
    by_key = {op[0]: op for op in ops}
    seq = [by_key[k] for (k, _, _) in order]
    defined = {("k", (0, 0, 0), m) for (_, _, m) in initial} | set(initial)
    remote_name = {}
    pos_def = {}
    # position at which every value becomes available
    for p, op in enumerate(seq):
        pos_def[op[0]] = p
    # read slot: `ahead` ops before use, not before the source is computed
    reads_at = {}
    for p, op in enumerate(seq):
        rem = op[4]
        if rem is None:
            continue
        (src, axis) = rem
        skey = ("k",) + src
        if sum(src[0]) == 0:
            earliest = 0
        else:
            earliest = pos_def[skey] + 1
        reads_at.setdefault(max(earliest, p - ahead), []).append((rem, skey))
    for p, op in enumerate(seq):
        issued = False
        for rem, skey in reads_at.get(p, []):
            if rem not in remote_name:
                remote_name[rem] = f"xr{len(remote_name)}"
                src, axis = rem
                lines.append(f"{ind}const double {remote_name[rem]} = {names.ket_remote(src, axis)};")
                issued = True
        if issued and PIN_REMOTE:
            lines.append(f"{ind}__builtin_amdgcn_sched_barrier(0x7);  // ALU may cross, LDS may not")
        rn = remote_name.get(op[4]) if op[4] is not None else None
        for l in op[3](rn):
            lines.append(f"{ind}{l}")




def _emit_hrr_scheduled(l1, l2, base_load, R, spherical, store, lines, ind, prefix, outputs=None,
                        preload=False):
    """HRR + transform of one column, emitted in liveness order.

    base_load(e) -> C expression reading base value (e, 0) (issued where first
    needed); store(k, expr) -> statement consuming output k.  ``outputs``, if
    given, restricts the column to those output indices and the values they
    depend on.  ``preload`` issues every base read first and waits for them
    once (empty asm statements that take the values as operands), instead of
    letting the compiler place each read just before its first use, which
    exposes the LDS latency at every read.
    """
    from .graph import schedule_min_live
    ops, base, outs = _hrr_ops(l1, l2, R, spherical)
    if outputs is not None:
        keep = {outs[i] for i in outputs}
        for k, terms in reversed(ops):
            if k in keep:
                keep.update(src for _, src in terms)
        ops = [(k, terms) for k, terms in ops if k in keep]
        base = [e for e in base if ("b", e) in keep]
        outs = [ok if i in set(outputs) else None for i, ok in enumerate(outs)]
    items = []
    code = {}
    names_ = {}

    def nm(k):
        return names_[k]
    for e in base:
        k = ("b", e)
        names_[k] = f"{prefix}b{len(names_)}"
        items.append((k, [], False))
        code[k] = (lambda k=k, e=e: f"const double {names_[k]} = {base_load(e)};")
    for i, (k, terms) in enumerate(ops):
        names_[k] = f"{prefix}o{i}"
        items.append((k, [src for _, src in terms], False))
        code[k] = (lambda k=k, terms=terms: f"const double {names_[k]} = " +
                   " + ".join(nm(src) if c is None else f"{c} * {nm(src)}" for c, src in terms) + ";")
    for i, ok in enumerate(outs):
        if ok is None:
            continue
        k = ("w", i)
        items.append((k, [ok], True))
        code[k] = (lambda i=i, ok=ok: store(i, nm(ok)))
    if preload:
        bn = [names_[("b", e)] for e in base]
        for e, x in zip(base, bn):
            lines.append(f"{ind}double {x} = {base_load(e)};")
        lines.append(f"{ind}{{  // every base value in registers before the recurrence starts")
        for i in range(0, len(bn), 8):
            ops_ = ", ".join(f'"+v"({x})' for x in bn[i:i + 8])
            lines.append(f'{ind}  asm volatile("" : {ops_});')
        lines.append(f"{ind}}}")
        items = [it for it in items if it[0][0] != "b"]
    for (k, ds, sink) in schedule_min_live(items, ()):
        lines.append(f"{ind}{code[k]()}")


REC_FIELDS = ["PAx", "PAy", "PAz", "WPx", "WPy", "WPz", "QCx", "QCy", "QCz", "WQx", "WQy", "WQz",
              "i2z", "i2e", "roz", "roe", "i2ze"]


UNIFORM_SCALARS = True


def _register_kernel(ci: ClassInfo, spherical: bool, k1: bool):
    """K4 = 1 kernel: persistent loop, next group's inputs prefetched.
    General kernel: one group of Q quartets per wave; the primitive quartets are
    set up in chunks of G -- each lane computes the geometry and Boys values of a
    different primitive quartet into LDS (field-major, so the writes are
    conflict-free and the group's reads are broadcasts) -- then the group runs the
    recurrence over the chunk."""
    kv = build_ket_vrr(ci.lc, ci.Lk)
    names = Names("V", kv, ci.Lk)
    G = ci.G
    Q = 64 // G
    NK = ci.nket(spherical)
    NEB = ci.n_ebra
    EOFF = ci.e_bra_offset
    BLK = ci.nout(spherical)
    cid = class_id(ci.la, ci.lb, ci.lc, ci.ld)
    tag = f"c{cid}_{'s' if spherical else 'c'}" + ("_k1" if k1 else "")
    lanes = ci.lanes
    lpos = {e: i for i, e in enumerate(lanes)}
    lane_tab = []
    for e in lanes:
        d = [lpos[sub(e, ax)] if e[ax] > 0 else -1 for ax in range(3)]
        lane_tab.append(e[0] | (e[1] << 4) | (e[2] << 8) | ((d[0] + 1) << 12) | ((d[1] + 1) << 18) | ((d[2] + 1) << 24))
    targets = kv.targets
    L = ci.L
    NREC = len(REC_FIELDS) + L + 1 + 2  # then constant rows 1.0 and 0.0 for the bra-path selectors
    use_rec = (not k1) and G > 1
    # LDS-selected bra-path factors pay off when the ket recurrence is short
    # (measured: faster for (xx|ss) and (ps|ps), slower once the ket phase's
    # cross-lane reads share the LDS pipeline)
    sel_lds = use_rec and SELECT_LDS_CONTRACTED and (ci.Lk == 0 or (ci.Lk == 1 and ci.Lb == 1))
    o = []
    o.append("namespace {")
    o.append(f"__constant__ int k_{tag}_lane[{G}] = {{" + ", ".join(str(v) for v in lane_tab) + "};")
    o.append("}  // namespace")
    o.append(f"__global__ void __launch_bounds__(64) eri_kernel_{tag}(EriClassArgs a)")
    o.append("{")
    o.append(f"  constexpr int G = {G}, Q = {Q}, NK = {NK}, NEB = {NEB}, BLK = {BLK};")
    # exchange rows, then one junk row that lanes without a bra output write to
    # (an LDS address with small positive offsets keeps the stores immediate-offset)
    o.append("  __shared__ double xch[Q * NEB * NK + NK];")
    o.append("  __shared__ double xab[Q * 3];")
    if use_rec:
        o.append(f"  constexpr int NREC = {NREC};")
        # odd field stride: lanes reading different fields of one record (the
        # bra-path selectors) hit different LDS banks
        o.append("  constexpr int RS = 65;")
        o.append("  __shared__ double rec[NREC * RS];  // field-major primitive-quartet records")
    o.append("  const int lane = threadIdx.x;")
    o.append("  int grp = lane / G, sub = lane - grp * G;")
    o.append("  if (grp >= Q) { grp = Q; sub = 0; }  // padding lanes: phantom group, e = (0,0,0)")
    o.append(f"  const int lt = k_{tag}_lane[sub];")
    o.append("  const int ex = lt & 15, ey = (lt >> 4) & 15, ez = (lt >> 8) & 15, es = ex + ey + ez;")
    o.append("  const int gb = grp * G;")
    o.append("  const int adx = (ex > 0 ? gb + ((lt >> 12) & 63) - 1 : lane) * 4;")
    o.append("  const int ady = (ey > 0 ? gb + ((lt >> 18) & 63) - 1 : lane) * 4;")
    o.append("  const int adz = (ez > 0 ? gb + ((lt >> 24) & 63) - 1 : lane) * 4;")
    o.append("  (void)adx; (void)ady; (void)adz; (void)es;")
    if sel_lds:
        o.append(f"  rec[{NREC - 2} * RS + lane] = 1.0;")
        o.append(f"  rec[{NREC - 1} * RS + lane] = 0.0;")
        _stage1_selectors(ci, o, "RS", NREC - 2, NREC - 1)
    o.append("  const int ngroups = (a.nq + Q - 1) / Q;")
    o.append("  int g = blockIdx.x;")
    o.append("  if (g >= ngroups) return;")
    o.append("  auto slot_of = [&](int gg) { int q = gg * Q + (grp < Q ? grp : 0); return q < a.nq ? q : a.nq - 1; };")
    o.append("  int qs = slot_of(g);")
    if k1 and Q == 1 and UNIFORM_SCALARS:
        o.append("  qs = __builtin_amdgcn_readfirstlane(qs);")
    o.append("  int bra = a.qbra[qs], ket = a.qket[qs];")
    o.append("  int4 pb = a.pair_info[bra], pk = a.pair_info[ket];")
    o.append("  for (;;) {")
    o.append("    const int gn = g + (int)gridDim.x;")
    if k1:
        if Q == 1 and UNIFORM_SCALARS:
            o.append("    const int qn = __builtin_amdgcn_readfirstlane(slot_of(gn < ngroups ? gn : g));")
        else:
            o.append("    const int qn = slot_of(gn < ngroups ? gn : g);")
        o.append("    const int bra_n = a.qbra[qn], ket_n = a.qket[qn];")
    o.append("    const double Ax = a.cen[3 * pb.x], Ay = a.cen[3 * pb.x + 1], Az = a.cen[3 * pb.x + 2];")
    o.append("    const double Cx = a.cen[3 * pk.x], Cy = a.cen[3 * pk.x + 1], Cz = a.cen[3 * pk.x + 2];")
    o.append("    const double CDx = Cx - a.cen[3 * pk.y], CDy = Cy - a.cen[3 * pk.y + 1], CDz = Cz - a.cen[3 * pk.y + 2];")
    o.append("    const double ABx = Ax - a.cen[3 * pb.y], ABy = Ay - a.cen[3 * pb.y + 1], ABz = Az - a.cen[3 * pb.y + 2];")
    o.append("    const double ACx = Ax - Cx, ACy = Ay - Cy, ACz = Az - Cz;")
    o.append("    (void)CDx; (void)CDy; (void)CDz;")

    def geom_lines(ind, pp_b, pp_k):
        r = []
        r.append(f"{ind}const EriPrimPair P = eri_load_pp(a.ppd, {pp_b});")
        r.append(f"{ind}const EriPrimPair K = eri_load_pp(a.ppd, {pp_k});")
        r.append(f"{ind}EriQuartetGeom gq;")
        r.append(f"{ind}eri_geom(P, K, ACx, ACy, ACz, gq);")
        r.append(f"{ind}double F[{L + 1}];")
        r.append(f"{ind}eri_boys<{L}>(gq.T, gq.pref, a.boys, F);")
        return r

    # one quartet per wave (K4 = 1 kernel): the quartet's scalars are the same
    # in every lane and move to scalar registers
    uni = k1 and Q == 1 and UNIFORM_SCALARS
    U = (lambda x: f"eri_uniform({x})") if uni else (lambda x: x)

    def scalars_from_geom(ind):
        r = []
        r.append(f"{ind}const double PAx = {U('P.PA[0]')}, PAy = {U('P.PA[1]')}, PAz = {U('P.PA[2]')};")
        r.append(f"{ind}const double WPx = {U('gq.WP[0]')}, WPy = {U('gq.WP[1]')}, WPz = {U('gq.WP[2]')};")
        r.append(f"{ind}const double QCx = {U('K.PA[0]')}, QCy = {U('K.PA[1]')}, QCz = {U('K.PA[2]')};")
        r.append(f"{ind}const double WQx = {U('gq.WQ[0]')}, WQy = {U('gq.WQ[1]')}, WQz = {U('gq.WQ[2]')};")
        r.append(f"{ind}const double i2z = {U('0.5 * P.izeta')}, i2e = {U('0.5 * K.izeta')}, roz = {U('gq.roz')}, "
                 f"roe = {U('gq.roe')}, i2ze = {U('gq.i2ze')};")
        return r

    init_keys = [("k", (0, 0, 0), m) for m in range(kv.base_m + 1)]

    def body(ind, with_acc, rsel=None):
        r = []
        r.append(f"{ind}const double ehx = ex * i2ze, ehy = ey * i2ze, ehz = ez * i2ze;")
        if rsel is None:
            r.append(f"{ind}(void)PAx; (void)PAy; (void)PAz; (void)WPx; (void)WPy; (void)WPz;")
        r.append(f"{ind}(void)QCx; (void)QCy; (void)QCz;")
        r.append(f"{ind}(void)WQx; (void)WQy; (void)WQz; (void)i2z; (void)i2e; (void)roz; (void)roe; (void)ehx; (void)ehy; (void)ehz;")
        _stage1(ci, kv.base_m, r, ind, rsel=rsel)
        if with_acc:
            _emit_scheduled(_lane_ops(ci, kv, names, spherical, False), init_keys, names, r, ind)
        else:
            r.append(f"{ind}double* xd = xch + ((grp < Q && es >= {ci.la}) ? (grp * NEB + (sub - {EOFF})) * NK : Q * NEB * NK);")
            _emit_scheduled(_lane_ops(ci, kv, names, spherical, True), init_keys, names, r, ind)
        return r

    tpos = {f: t for t, (f, m) in enumerate(targets)}
    if k1:
        o.append("    {")
        o += geom_lines("      ", "pb.z", "pk.z")
        o += scalars_from_geom("      ")
        o += body("      ", False)
        base_of = None
        hind = "      "
    elif not use_rec:
        for t in range(len(targets)):
            o.append(f"    double acc{t} = 0.0;")
        o.append("    for (int ib = 0; ib < pb.w; ++ib) {")
        o.append("      for (int ik = 0; ik < pk.w; ++ik) {")
        o += geom_lines("        ", "pb.z + ib", "pk.z + ik")
        o += scalars_from_geom("        ")
        o += body("        ", True)
        o.append("      }")
        o.append("    }")
        base_of = lambda e: f"acc{tpos[e]}"
        hind = "    "
    else:
        for t in range(len(targets)):
            o.append(f"    double acc{t} = 0.0;")
        o.append("    const int K4 = pb.w * pk.w;")
        o.append("    for (int c0 = 0; c0 < K4; c0 += G) {")
        o.append("      {  // this lane's primitive quartet of the chunk -> LDS record")
        o.append("        const int t = c0 + sub < K4 ? c0 + sub : K4 - 1;")
        o.append("        const int ib = t / pk.w, ik = t - ib * pk.w;")
        o += geom_lines("        ", "pb.z + ib", "pk.z + ik")
        vals = ["P.PA[0]", "P.PA[1]", "P.PA[2]", "gq.WP[0]", "gq.WP[1]", "gq.WP[2]", "K.PA[0]", "K.PA[1]", "K.PA[2]",
                "gq.WQ[0]", "gq.WQ[1]", "gq.WQ[2]", "0.5 * P.izeta", "0.5 * K.izeta", "gq.roz", "gq.roe", "gq.i2ze"]
        o.append("        double* r = rec + lane;")
        for fi, v in enumerate(vals):
            o.append(f"        r[{fi} * RS] = {v};")
        for m in range(L + 1):
            o.append(f"        r[{len(vals) + m} * RS] = F[{m}];")
        o.append("      }")
        o.append("      __syncthreads();")
        o.append("      const int n = K4 - c0 < G ? K4 - c0 : G;")
        o.append("      for (int j = 0; j < n; ++j) {")
        o.append("        const double* r = rec + gb + j;")
        for fi, nm in enumerate(REC_FIELDS):
            if fi >= 6 or not sel_lds:  # P-A and W-P: read by the bra path through its selectors
                o.append(f"        const double {nm} = r[{fi} * RS];")
        o.append(f"        double F[{L + 1}];")
        for m in range(L + 1):
            o.append(f"        F[{m}] = r[{len(REC_FIELDS) + m} * RS];")
        o += body("        ", True, rsel="r" if sel_lds else None)
        o.append("      }")
        o.append("      __syncthreads();  // records are rewritten by the next chunk")
        o.append("    }")
        base_of = lambda e: f"acc{tpos[e]}"
        hind = "    "
    if not k1:
        # H1: ket HRR + transform per lane on the contracted values
        o.append(f"{hind}double* yd = xch + ((grp < Q && es >= {ci.la}) ? (grp * NEB + (sub - {EOFF})) * NK : Q * NEB * NK);")
        _emit_hrr_scheduled(ci.lc, ci.ld, base_of, "CD", spherical, lambda k, x: f"yd[{k}] = {x};", o, hind, "y")
    o.append(f"{hind}if (grp < Q && sub == 0) {{ xab[3 * grp] = ABx; xab[3 * grp + 1] = ABy; xab[3 * grp + 2] = ABz; }}")
    if k1:
        o.append("    }")
    o.append("    __syncthreads();")
    if k1:
        o.append("    const int4 pb_n = a.pair_info[bra_n], pk_n = a.pair_info[ket_n];")
    # H2: lanes own ket components
    o.append("    const int q0 = g * Q;")
    o.append("    for (int t = lane; t < Q * NK; t += 64) {")
    o.append("      const int g2 = t / NK, kap = t - g2 * NK;")
    o.append("      const int slot = q0 + g2;")
    o.append("      if (slot >= a.nq) continue;")
    o.append("      const double ABx = xab[3 * g2], ABy = xab[3 * g2 + 1], ABz = xab[3 * g2 + 2];")
    o.append("      (void)ABx; (void)ABy; (void)ABz;")
    o.append("      const double* src = xch + g2 * NEB * NK + kap;")
    ebra = [e for l in range(ci.la, ci.Lb + 1) for e in components(l)]
    epos = {e: i for i, e in enumerate(ebra)}
    o.append("      double* dst = a.out + (size_t)slot * BLK + kap;")
    _emit_hrr_scheduled(ci.la, ci.lb, lambda e: f"src[{epos[e]} * NK]", "AB", spherical,
                        lambda k, x: f"eri_out(&dst[{k} * NK], {x});", o, "      ", "z")
    o.append("    }")
    o.append("    if (gn >= ngroups) break;")
    o.append("    __syncthreads();  // exchange buffer reused by the next group")
    if k1:
        o.append("    g = gn; qs = qn; bra = bra_n; ket = ket_n; pb = pb_n; pk = pk_n;")
    else:
        o.append("    g = gn; qs = slot_of(g); bra = a.qbra[qs]; ket = a.qket[qs];")
        o.append("    pb = a.pair_info[bra]; pk = a.pair_info[ket];")
    o.append("  }")
    o.append("}")
    o.append("")
    o.append(f"void eri_launch_{tag}(const EriClassArgs& a, hipStream_t s)")
    o.append("{")
    o.append(f"  const int ngroups = (a.nq + {Q} - 1) / {Q};")
    if k1:
        o.append("  const int nblk = ngroups < a.grid_cap ? ngroups : a.grid_cap;")
    else:
        o.append("  const int nblk = ngroups;  // one group per workgroup")
    o.append(f"  if (nblk > 0) hipLaunchKernelGGL(eri_kernel_{tag}, dim3(nblk), dim3(64), 0, s, a);")
    o.append("}")
    o.append("")
    return o


def tier_of(ci: ClassInfo, spherical: bool = True) -> str:
    """Register tier whenever a lane group fits one wave (the compiler may keep
    part of a large live set in AGPRs), the class fits the one-quartet-per-lane
    tier, or a wider group runs packed; memory tier for the other wider bra
    groups.  The tier can depend on the output kind (``spherical``).  The
    single-tier ablation variants route every class to one tier."""
    from .variant import CURRENT
    from .lane import use_lane_tier
    from .packed import wide_packed
    if CURRENT.tiers == "memory":
        return "M"
    if CURRENT.tiers == "lane":
        return "V"
    if ci.G > 64 and use_lane_tier(ci, True):
        return "V"  # a wide bra with an s-type ket, small enough for one quartet per lane
    if ci.Lb == 5 and ci.Lk >= 5 and not use_lane_tier(ci, True):
        # 56-lane bras with long ket recurrences: the memory tier measured 15-20%
        # faster ((fd|fd): 3.46 -> 2.94 ms for a K = 2 batch); with shorter kets
        # it measured 20-60% slower
        return "M"
    if wide_packed(ci, spherical):
        return "V"  # 84- and 120-lane bras with short kets: packed multi-wave workgroups
    return "V" if ci.G <= 64 else "M"


def generate(out_dir: str, lmax: int = 4, classes=None, cartesian_only=()):
    """Write one .hip per (class, output kind) plus the dispatch table; the
    classes in ``cartesian_only`` (the raised-shell classes of the derivative
    integrals, which run on raw Cartesian monomials) get the Cartesian kind only."""
    from .graph import all_classes
    os.makedirs(out_dir, exist_ok=True)
    cls = list(classes if classes is not None else all_classes(lmax))
    cart_only = list(cartesian_only)
    entries = []
    files = []
    for ci in cls + cart_only:
        for spherical in ((False,) if ci in cart_only else (False, True)):
            tier = tier_of(ci, spherical)
            if tier == "V":
                src = emit_register_tier(ci, spherical)
            else:
                src = emit_memory_tier(ci, spherical)
            cid = class_id(ci.la, ci.lb, ci.lc, ci.ld)
            tag = f"c{cid}_{'s' if spherical else 'c'}"
            fn = os.path.join(out_dir, f"eri_{tag}.hip")
            _write_if_changed(fn, src)
            files.append(fn)
            entries.append((cid, spherical, tag, tier, ci))
    # dispatch
    d = ['#include "eri_device.h"', ""]
    for cid, sph, tag, tier, ci in entries:
        d.append(f"void eri_launch_{tag}(const EriClassArgs& a, hipStream_t s);")
        if tier == "V":
            d.append(f"void eri_launch_{tag}_k1(const EriClassArgs& a, hipStream_t s);")
    d.append("")
    d.append("EriClassEntry eri_class_table[] = {")
    for cid, sph, tag, tier, ci in entries:
        scr = memory_tier_scratch_doubles(ci, sph) if tier == "M" else 0
        k1 = f"eri_launch_{tag}_k1" if tier == "V" else f"eri_launch_{tag}"
        d.append(f"  {{{cid}, {1 if sph else 0}, {ci.la}, {ci.lb}, {ci.lc}, {ci.ld}, '{tier}', {scr}, eri_launch_{tag}, {k1}}},")
    d.append("};")
    d.append(f"const int eri_class_table_size = {len(entries)};")
    fn = os.path.join(out_dir, "eri_dispatch.hip")
    _write_if_changed(fn, "\n".join(d) + "\n")
    files.append(fn)
    _write_if_changed(os.path.join(out_dir, "eri_sph_table.h"), sph_table_header())
    return files, entries


def sph_table_header(lmax: int = 4) -> str:
    """t^(l) for l <= lmax as a device constant table (row m = -l..l over the
    Cartesian components, row-major, each l padded to a common stride), for the
    runtime's transform of derivative blocks."""
    from .cartesian import sph_matrix, ncart as nc_, nsph as ns_
    stride = ns_(lmax) * nc_(lmax)
    lines = ["// generated: real solid harmonic transforms t^(l), rows m = -l..l over Cartesian components",
             "#pragma once", f"#define ERI_SPH_STRIDE {stride}",
             f"static __constant__ double eri_sph_T[{lmax + 1}][{stride}] = {{"]
    for l in range(lmax + 1):
        vals = [v for row in sph_matrix(l) for v in row]
        vals += [0.0] * (stride - len(vals))
        lines.append("  {" + ", ".join(repr(float(v)) for v in vals) + "},")
    lines.append("};")
    return "\n".join(lines) + "\n"


def _write_if_changed(fn, text):
    if os.path.exists(fn):
        with open(fn) as f:
            if f.read() == text:
                return
    with open(fn, "w") as f:
        f.write(text)


# ---------------------------------------------------------------------------
# memory tier
# ---------------------------------------------------------------------------

def _count_private(ops, outs):
    lines = []
    return _emit_ops_mem(ops, lambda e: "0.0", outs, lambda i, x: f"(void)({x});", 0, lines, "")


def _coupling_levels(kv):
    """Per ket level k >= 1: the values of level k-1 read across lanes by level k."""
    levels = {}
    for n in kv.nodes:
        levels.setdefault(sum(n.f), [])
        if n.a1 not in levels[sum(n.f)]:
            levels[sum(n.f)].append(n.a1)
    return levels


def mem_lds_doubles(ci: ClassInfo) -> int:
    kv = build_ket_vrr(ci.lc, ci.Lk)
    W = 64 * ((ci.G + 63) // 64)
    lv = _coupling_levels(kv)
    return (max((len(v) for v in lv.values()), default=0)) * W


def mem_acc_in_registers(ci: ClassInfo) -> bool:
    """Memory tier: keep the contraction accumulators in registers when they
    fit beside the ket recurrence's live set (VGPRs + AGPRs at occupancy 1)."""
    kv = build_ket_vrr(ci.lc, ci.Lk)
    live = ket_vrr_peak_live(kv) if kv.nodes else 0
    return live + len(kv.targets) <= 170


def _mem_layout(ci: ClassInfo, spherical: bool):
    """Scratch rows (units of W doubles): only the contraction accumulators of
    classes whose accumulators do not fit in registers."""
    kv = build_ket_vrr(ci.lc, ci.Lk)
    nslots = 0 if mem_acc_in_registers(ci) else len(kv.targets)
    if not mem_xch_in_lds(ci, spherical):
        nslots += ci.nket(spherical)  # exchange rows follow the accumulators
    W = 64 * ((ci.G + 63) // 64)
    return kv, nslots, W


LDS_LIMIT_BYTES = 160 * 1024
# primitive quartets set up together (one lane each) into LDS records
MEM_CHUNK = 32
# memory-tier classes with a ket of total angular momentum up to this run at two waves per SIMD
MEM_TWO_WAVES_MAX_LK = 4


def mem_rec_fields(ci: ClassInfo) -> int:
    """Fields of one primitive-quartet record: P-A, W-P, Q-C, W-Q, 1/(2 zeta),
    1/(2 eta), rho/zeta, rho/eta, 1/(2(zeta+eta)), then F_0..F_L."""
    return 17 + ci.L + 1


def mem_rec_bytes(ci: ClassInfo) -> int:
    return 8 * mem_rec_fields(ci) * (MEM_CHUNK | 1)


def mem_xch_in_lds(ci: ClassInfo, spherical: bool) -> bool:
    return ci.nket(spherical) * mem_xch_stride(ci) * 8 + mem_rec_bytes(ci) <= LDS_LIMIT_BYTES


def mem_xch_stride(ci: ClassInfo) -> int:
    """Row stride (doubles) of the LDS exchange: W + 1, so that lanes reading
    different rows at one column hit different banks."""
    return 64 * ((ci.G + 63) // 64) + 1


def mem_lds_total(ci: ClassInfo, spherical: bool) -> int:
    """LDS doubles: the ket level buffer and the exchange share one array."""
    xch = ci.nket(spherical) * mem_xch_stride(ci) if mem_xch_in_lds(ci, spherical) else 0
    return max(1, mem_lds_doubles(ci), xch)


def memory_tier_scratch_doubles(ci: ClassInfo, spherical: bool) -> int:
    """Global scratch doubles per workgroup (0 when the accumulators are registers)."""
    kv, nslots, W = _mem_layout(ci, spherical)
    return nslots * W


def emit_memory_tier(ci: ClassInfo, spherical: bool) -> str:
    kv, nslots, W = _mem_layout(ci, spherical)
    acc0 = 0
    XS = mem_xch_stride(ci)
    xlds = mem_xch_in_lds(ci, spherical)
    xch0 = nslots - ci.nket(spherical)  # first exchange row when it lives in scratch
    names = Names("V", kv, ci.Lk)
    G = ci.G
    NK = ci.nket(spherical)
    NEB = ci.n_ebra
    EOFF = ci.e_bra_offset
    BLK = ci.nout(spherical)
    cid = class_id(ci.la, ci.lb, ci.lc, ci.ld)
    tag = f"c{cid}_{'s' if spherical else 'c'}"
    lanes = ci.lanes
    lpos = {e: i for i, e in enumerate(lanes)}
    tx = [e[0] for e in lanes]
    ty = [e[1] for e in lanes]
    tz = [e[2] for e in lanes]
    dx = [lpos[sub(e, 0)] if e[0] > 0 else -1 for e in lanes]
    dy = [lpos[sub(e, 1)] if e[1] > 0 else -1 for e in lanes]
    dz = [lpos[sub(e, 2)] if e[2] > 0 else -1 for e in lanes]
    targets = kv.targets
    L = ci.L
    o = []
    o.append(f"// class ({ci.la}{ci.lb}|{ci.lc}{ci.ld}) id {cid}, {'spherical' if spherical else 'Cartesian'} output,"
             f" memory tier: {G} lanes (workgroup {W}) per quartet, {nslots} scratch rows")
    o.append('#include "eri_device.h"')
    o.append("namespace {")
    o.append(f"__constant__ short k_{tag}_lane[3][{G}] = {{")
    for arr in (tx, ty, tz):
        o.append("  {" + ", ".join(str(v) for v in arr) + "},")
    o.append("};")
    o.append(f"__constant__ short k_{tag}_down[3][{G}] = {{")
    for arr in (dx, dy, dz):
        o.append("  {" + ", ".join(str(v) for v in arr) + "},")
    o.append("};")
    o.append("}  // namespace")
    o.append("")
    # short ket recurrences: two waves per SIMD (at most 256 registers, a few
    # spilled values) measured 20-25% faster than one wave with no spill for
    # kets up to l = 4 in total, and 15% slower for (ff|fd)
    lb = f"{W}, 2" if ci.Lk <= MEM_TWO_WAVES_MAX_LK else f"{W}"
    o.append(f"__global__ void __launch_bounds__({lb}) eri_kernel_{tag}(EriClassArgs a)")
    o.append("{")
    o.append(f"  constexpr int G = {G}, W = {W}, NK = {NK}, NEB = {NEB}, BLK = {BLK};")
    o.append(f"  constexpr size_t WG_DOUBLES = {memory_tier_scratch_doubles(ci, spherical)};")
    o.append("  const int tid = threadIdx.x;")
    # one LDS array: a ket level's cross-lane values during the recurrence,
    # then the ket-transformed exchange (row kappa, column = bra lane)
    o.append(f"  __shared__ double xl[{mem_lds_total(ci, spherical)}];")
    o.append(f"  constexpr int XS = {XS};")
    NRM = mem_rec_fields(ci)
    o.append(f"  constexpr int CHM = {MEM_CHUNK}, RSM = {MEM_CHUNK | 1};")
    o.append(f"  __shared__ double mrec[{NRM} * RSM];  // field-major records of one chunk of primitive quartets")
    o.append("  const int sub = tid < G ? tid : 0;  // lanes beyond G shadow e = (0,0,0) and never store")
    o.append("  const bool real = tid < G;")
    # Every graph value lives in this workgroup's scratch slice, addressed by
    # buffer instructions: one per-lane VGPR offset plus a uniform slot offset,
    # so the thousands of slots cost no address registers.
    o.append("  double* slice = a.scratch + (size_t)blockIdx.x * WG_DOUBLES;")
    o.append("  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(slice, (short)0, (int)(WG_DOUBLES * 8), 0x00020000);")
    o.append("  const int vo = tid * 8;")
    o.append("#define SLD(s) eri_bld(rs, vo, (s) * (W * 8))")
    o.append("#define SST(s, x) eri_bst(rs, vo, (s) * (W * 8), (x))")
    o.append("#define SLDL(s, l) eri_bld(rs, (l) * 8, (s) * (W * 8))")
    o.append(f"  const int ex = k_{tag}_lane[0][sub], ey = k_{tag}_lane[1][sub], ez = k_{tag}_lane[2][sub];")
    o.append("  const int es = ex + ey + ez;")
    o.append(f"  const int srcx = ex > 0 ? k_{tag}_down[0][sub] : tid;")
    o.append(f"  const int srcy = ey > 0 ? k_{tag}_down[1][sub] : tid;")
    o.append(f"  const int srcz = ez > 0 ? k_{tag}_down[2][sub] : tid;")
    o.append("  (void)srcx; (void)srcy; (void)srcz; (void)real;")
    o.append("  for (int qs = blockIdx.x; qs < a.nq; qs += gridDim.x) {")
    o.append("  const int bra = a.qbra[qs], ket = a.qket[qs];")
    o.append("  const int4 pb = a.pair_info[bra], pk = a.pair_info[ket];")
    o.append("  const double Cx = a.cen[3 * pk.x], Cy = a.cen[3 * pk.x + 1], Cz = a.cen[3 * pk.x + 2];")
    o.append("  const double CDx = Cx - a.cen[3 * pk.y], CDy = Cy - a.cen[3 * pk.y + 1], CDz = Cz - a.cen[3 * pk.y + 2];")
    o.append("  const double ACx = a.cen[3 * pb.x] - Cx, ACy = a.cen[3 * pb.x + 1] - Cy, ACz = a.cen[3 * pb.x + 2] - Cz;")
    o.append("  (void)CDx; (void)CDy; (void)CDz;")
    acc_reg = mem_acc_in_registers(ci)
    if acc_reg:
        for t in range(len(targets)):
            o.append(f"  double acc{t} = 0.0;")
    else:
        for t in range(len(targets)):
            o.append(f"  SST({acc0 + t}, 0.0);")
    # primitive quartets in chunks of CHM: lane t < CHM sets up primitive
    # quartet c0 + t (geometry and Boys values) into an LDS record, then every
    # lane evaluates the chunk's primitive quartets one after another from
    # the records (broadcast reads), instead of every lane repeating the set-up
    rec_vals = ["P.PA[0]", "P.PA[1]", "P.PA[2]", "gq.WP[0]", "gq.WP[1]", "gq.WP[2]", "K.PA[0]", "K.PA[1]", "K.PA[2]",
                "gq.WQ[0]", "gq.WQ[1]", "gq.WQ[2]", "0.5 * P.izeta", "0.5 * K.izeta", "gq.roz", "gq.roe",
                "gq.i2ze"] + [f"Fq[{m}]" for m in range(L + 1)]
    rec_names = ["PAx", "PAy", "PAz", "WPx", "WPy", "WPz", "QCx", "QCy", "QCz", "WQx", "WQy", "WQz",
                 "i2z", "i2e", "roz", "roe", "i2ze"]
    assert len(rec_vals) == NRM
    o.append("  const int K4 = pb.w * pk.w;")
    o.append("  for (int c0 = 0; c0 < K4; c0 += CHM) {")
    o.append("    if (tid < CHM && c0 + tid < K4) {")
    o.append("      const int p = c0 + tid, ib = p / pk.w, ik = p - ib * pk.w;")
    o.append("      const EriPrimPair P = eri_load_pp(a.ppd, pb.z + ib);")
    o.append("      const EriPrimPair K = eri_load_pp(a.ppd, pk.z + ik);")
    o.append("      EriQuartetGeom gq;")
    o.append("      eri_geom(P, K, ACx, ACy, ACz, gq);")
    o.append(f"      double Fq[{L + 1}];")
    o.append(f"      eri_boys<{L}>(gq.T, gq.pref, a.boys, Fq);")
    o.append("      double* r = mrec + tid;")
    for fi, v in enumerate(rec_vals):
        o.append(f"      r[{fi} * RSM] = {v};")
    o.append("    }")
    o.append("    __syncthreads();  // the chunk's records are written")
    o.append("    const int nch = K4 - c0 < CHM ? K4 - c0 : CHM;")
    o.append("    for (int j = 0; j < nch; ++j) {")
    o.append("      const double* r = mrec + j;")
    for fi, nm in enumerate(rec_names):
        o.append(f"      const double {nm} = r[{fi} * RSM];")
    o.append("      const double ehx = ex * i2ze, ehy = ey * i2ze, ehz = ez * i2ze;")
    o.append("      (void)PAx; (void)PAy; (void)PAz; (void)WPx; (void)WPy; (void)WPz; (void)QCx; (void)QCy; (void)QCz;")
    o.append("      (void)WQx; (void)WQy; (void)WQz; (void)i2z; (void)i2e; (void)roz; (void)roe; (void)ehx; (void)ehy; (void)ehz;")
    o.append(f"      double F[{L + 1}];")
    for m in range(L + 1):
        o.append(f"      F[{m}] = r[{17 + m} * RSM];")
    # without the first-step shortcut: with it the spilling memory-tier kernels
    # measured slower ((gg|gg) x 1000 at K = 2: 2.24 against 2.04 ms)
    _stage1(ci, kv.base_m, o, shortcut=False)
    # ket phase: own values in registers (level order); the coupling operand of
    # level k is read from an LDS buffer holding level k-1's cross-lane values
    lv = _coupling_levels(kv)

    def acc_add(t, val):
        if acc_reg:
            o.append(f"      acc{t} += {val};")
        else:
            o.append(f"      SST({acc0 + t}, ap{t} + {val});")

    def acc_fetch(ts):
        # scratch accumulators of one level are read in one batch, before the
        # level's barrier, so that their latency overlaps it
        if not acc_reg:
            for t in ts:
                o.append(f"      const double ap{t} = SLD({acc0 + t});")

    tpos_all = {tg: t for t, tg in enumerate(targets)}
    base_t = [t for t, tg in enumerate(targets) if sum(tg[0]) == 0]
    acc_fetch(base_t)
    for t in base_t:
        acc_add(t, f"s1_{targets[t][1]}")
    levels = sorted({sum(n.f) for n in kv.nodes})
    for k in levels:
        acc_fetch([t for t, tg in enumerate(targets) if sum(tg[0]) == k])
        # publish level k-1 values that level k reads across lanes
        o.append("      __syncthreads();")
        for j, key in enumerate(lv[k]):
            val = f"s1_{key[1]}" if sum(key[0]) == 0 else names.ket(key)
            o.append(f"      xl[{j} * W + tid] = {val};")
        o.append("      __syncthreads();")
        for n in kv.nodes:
            if sum(n.f) != k:
                continue
            a = AX[n.axis]
            j = lv[k].index(n.a1)
            expr = f"QC{a} * {names.ket(n.a0)} + WQ{a} * {names.ket(n.a1)}"
            if n.b0 is not None:
                expr += f" + {_fmt(n.fi_minus_1)} * i2e * ({names.ket(n.b0)} - roe * {names.ket(n.b1)})"
            expr += f" + eh{a} * xl[{j} * W + src{a}]"
            o.append(f"      const double {names.ket((n.f, n.m))} = {expr};")
            if (n.f, n.m) in tpos_all:
                acc_add(tpos_all[(n.f, n.m)], names.ket((n.f, n.m)))
    o.append("      __syncthreads();  // all reads of this primitive quartet (records, level slots) done")
    o.append("    }")
    o.append("  }")
    # ket HRR and transform per lane, in registers, from the accumulators;
    # results into the LDS exchange (the last barrier of the loop freed it)
    tpos = {f: t for t, (f, m) in enumerate(targets)}
    acc_src = (lambda e: f"acc{tpos[e]}") if acc_reg else (lambda e: f"SLD({acc0 + tpos[e]})")
    o.append("  {")
    if xlds:
        h1_store = lambda k, x: f"xl[{k} * XS + tid] = {x};"
    else:
        h1_store = lambda k, x: f"SST({xch0 + k}, {x});"
    _emit_hrr_scheduled(ci.lc, ci.ld, acc_src, "CD", spherical, h1_store, o, "    ", "h")
    o.append("  }")
    o.append("  __syncthreads();")
    o.append("  const int4 pb2 = a.pair_info[bra];")
    o.append("  const double ABx = a.cen[3 * pb2.x] - a.cen[3 * pb2.y], ABy = a.cen[3 * pb2.x + 1] - a.cen[3 * pb2.y + 1],"
             " ABz = a.cen[3 * pb2.x + 2] - a.cen[3 * pb2.y + 2];")
    o.append("  (void)ABx; (void)ABy; (void)ABz;")
    # bra HRR and transform per ket component kappa, in registers
    o.append("  for (int kap = tid; kap < NK; kap += W) {")
    ebra = [e for l in range(ci.la, ci.Lb + 1) for e in components(l)]
    epos = {e: i for i, e in enumerate(ebra)}
    o.append("    double* dst = a.out + (size_t)qs * BLK + kap;")
    if xlds:
        o.append(f"    const double* xr = xl + kap * XS + {EOFF};  // exchange row kappa, first bra lane")
        h2_load = lambda e: f"xr[{epos[e]}]"
    else:
        o.append(f"    const int vx = (kap * W + {EOFF}) * 8;  // exchange row kappa, first bra lane")
        h2_load = lambda e: f"eri_bld(rs, vx, {xch0} * (W * 8) + {epos[e] * 8})"
    _emit_hrr_scheduled(ci.la, ci.lb, h2_load, "AB", spherical,
                        lambda k, x: f"eri_out(&dst[{k} * NK], {x});", o, "    ", "g")
    o.append("  }")
    o.append("  __syncthreads();  // the exchange is reused by the next quartet")
    o.append("  }")
    o.append("#undef SLD")
    o.append("#undef SST")
    o.append("#undef SLDL")
    o.append("}")
    o.append("")
    o.append(f"void eri_launch_{tag}(const EriClassArgs& a, hipStream_t s)")
    o.append("{")
    o.append("  const int nblk = a.nq < ERI_MEM_WGS ? a.nq : ERI_MEM_WGS;")
    o.append(f"  if (nblk > 0) hipLaunchKernelGGL(eri_kernel_{tag}, dim3(nblk), dim3({W}), 0, s, a);")
    o.append("}")
    return "\n".join(o) + "\n"
