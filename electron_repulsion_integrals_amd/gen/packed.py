"""Packed register-tier kernels: several quartets per multi-wave workgroup.

The register tier maps one bra component e to one lane, so a quartet occupies
G = #{e : |e| <= la+lb} lanes.  When G does not divide 64 (G = 35 for a bra
of total angular momentum 4, e.g. the (dd| and (fp| classes), a wave64 holds
one quartet and a large share of its lanes idles through every phase.  Here a
workgroup of W waves holds Q = floor(64 W / G) quartets back to back (lane t
serves quartet t / G, component t mod G), so the lanes are almost all busy.

The coupling operand of the ket recurrence, [e-1_i 0|f-1_i 0]^(m+1), may then
belong to another wave.  The ket recurrence therefore runs level by level
(level k = nodes with |f| = k): each lane publishes the values of level k-1
that level k reads across lanes to an LDS buffer, one workgroup barrier, and
every lane reads its coupling operands for the whole level at once.  Two
buffers alternate, so one barrier per level suffices.  On gfx950 this is also
cheaper than the wave-local ds_bpermute it replaces: a double via bpermute is
two permute instructions at about 6 LDS clocks each, against one 64-bit LDS
read (about 4 clocks) plus a share of one 64-bit write that serves every
reader of that value.

Algorithmically nothing changes ("FusionRCG", section II-A, Eq. (2) and its ket
twin for the vertical recurrence, Eq. (3) for the horizontal ones, Eq. (14)
for the stepwise spherical transform): per quartet the lanes walk the bra
path, run the ket recurrence, apply the ket HRR and transform per lane, hand
the block through one LDS exchange to lanes that own ket components, and
finish with the bra HRR and transform.
"""
from __future__ import annotations

import functools

from .cartesian import components, sub
from .graph import ClassInfo, build_ket_vrr, class_id

LDS_BYTES = 160 * 1024
# measured on the (dd|dd) batch: two waves (three quartets) per workgroup beat
# three or four waves; a record batch covering eight groups
PACK_WAVES = 2
PACK_RB = 8


def wide_packed(ci: ClassInfo, spherical: bool = False) -> bool:
    """Lane groups wider than a wave with a ket recurrence of total angular
    momentum 1..5 run both kernels as packed multi-wave workgroups instead of
    going to the memory tier:
      84-lane bras (la + lb = 6: (ff|, (gd|): three quartets on four waves
        (252 of 256 lanes).  Measured on the 120-atom cluster: (ff|ps) .. (ff|fp)
        1.5-1.9x faster, (ff|fd) 17% faster even at one workgroup per compute
        unit.  With an l = 6 ket only the spherical kernels fit a compute unit's
        LDS (the Cartesian K4 = 1 kernel would need 186 KB); spherical (ff|ff)
        measured 1.16x faster than in the memory tier (4,000 quartets, K = 2).
      120-lane bras (la + lb = 7: (gf|): one quartet on two waves (120 of 128
        lanes).  Measured on K = 2 batches: 1.34-1.40x faster with p and d kets,
        1.17-1.24x with l = 4 and (gf|gp), 1.03x with (gf|fd); l = 6 kets tie
        and stay in the memory tier.
      165-lane bras ((gg|) with kets up to l = 4: one quartet on three waves
        (165 of 192 lanes).  Measured: 1.56-2.94x faster on K = 2 batches,
        1.18-2.63x on K = 1 batches."""
    if ci.G == 84 and ci.Lk == 6:
        return spherical
    if ci.G == 165:
        return 1 <= ci.Lk <= 4
    return ci.G in (84, 120) and 1 <= ci.Lk <= 5


def _wide_waves(ci: ClassInfo) -> int:
    return {84: 4, 165: 3}.get(ci.G, 2)


def packed_k1_waves(ci: ClassInfo, spherical: bool = True) -> int:
    if _k1_three(ci, spherical):
        return K1_THREE_WAVES_W
    return _wide_waves(ci) if ci.G > 64 else PACK_WAVES


# K4 = 1 kernels built for three waves per SIMD instead of two, on workgroups
# of three waves (five 35-lane quartets in 192 lanes).  Their bra-path
# selectors are packed one int per step, which keeps (dd|dd) at 164 VGPRs
# with no scratch, and a record batch of five groups fits four workgroups in
# a compute unit's LDS.  Measured on the (dd|dd) batch against two waves per
# SIMD: three waves per SIMD 5% faster, the five-group record batch (no reload
# within a 20,000-quartet batch) 2% more, three-wave workgroups 1.5% more.
K1_THREE_WAVES = {(2, 2, 2, 2, True)}  # (la, lb, lc, ld, spherical)
K1_THREE_WAVES_RB = 5
K1_THREE_WAVES_W = 3


def _k1_three(ci: ClassInfo, spherical: bool) -> bool:
    return (ci.la, ci.lb, ci.lc, ci.ld, spherical) in K1_THREE_WAVES and ci.G <= 64


def _k1_waves_per_simd(ci: ClassInfo, spherical: bool) -> int:
    return 3 if _k1_three(ci, spherical) else 2


def _k1_rb(ci: ClassInfo, spherical: bool) -> int:
    return K1_THREE_WAVES_RB if _k1_three(ci, spherical) else PACK_RB


def packed_k1_min_waves(ci: ClassInfo, spherical: bool = True) -> int:
    """Occupancy bound of the K4 = 1 kernel (0: the compiler's choice).  84-lane
    bras with kets up to l = 4 otherwise take 56-62 AGPRs beyond 256 VGPRs and
    run at one wave per SIMD; capped at two they measured 1.15-1.39x faster for
    (ff|ps) .. (ff|fp) on K = 1 batches and even for (gd| apart from (gd|fp)
    (1.22x).  The cap made the 120-lane kernels slower."""
    if _k1_three(ci, spherical):
        return 3
    return 2 if wide_packed(ci) and ci.G == 84 and ci.Lk <= 4 else 0


def packed_shape(ci: ClassInfo, spherical: bool, waves: int = PACK_WAVES):
    """(W, Q, NT): waves per workgroup, quartets per workgroup, threads."""
    NT = 64 * waves
    return waves, NT // ci.G, NT


def _levels(kv):
    """Per ket level k: the distinct coupling sources (values of level k-1)."""
    lv = {}
    for n in kv.nodes:
        lst = lv.setdefault(sum(n.f), [])
        if n.a1 not in lst:
            lst.append(n.a1)
    return lv


# The exchange rows of the bra HRR lie apart from the last ket level's buffer,
# so the exchange can be written right after that level's reads without a
# second barrier; the levels before alternate between the start of the buffer
# and the offset past the exchange.  Kept only where the larger buffer leaves
# as many workgroups per compute unit.
XD_APART = True


def _level_buffers(ci: ClassInfo, spherical: bool, waves: int, apart: bool):
    """(offset of each ket level's buffer in doubles, doubles of the whole
    buffer).  Level k's buffer may not overlap level k-1's (a lane can publish
    level k while another still reads level k-1); with ``apart`` the exchange
    rows (written after the last level's reads) do not overlap the last
    level's buffer."""
    kv = build_ket_vrr(ci.lc, ci.Lk)
    W, Q, NT = packed_shape(ci, spherical, waves)
    lv = _levels(kv)
    levels = sorted(lv)
    NC = max((len(v) for v in lv.values()), default=0)
    NX = Q * ci.n_ebra * ci.nket(spherical) + ci.nket(spherical)
    if not apart:
        # levels of even index at the start, odd ones after the widest even one
        ne = max((len(lv[k]) for li, k in enumerate(levels) if li % 2 == 0), default=0)
        no = max((len(lv[k]) for li, k in enumerate(levels) if li % 2 == 1), default=0)
        return [(li % 2) * ne * NT for li in range(len(levels))], max((ne + no) * NT, NX)
    far = max(NX, NC * NT)
    nl = len(levels)
    offs = [far if (nl - 1 - li) % 2 == 0 else 0 for li in range(nl)]
    size = max([NX] + [offs[li] + len(lv[k]) * NT for li, k in enumerate(levels)])
    return offs, size


def _lds_bytes(ci, spherical, waves, rb, apart):
    W, Q, NT = packed_shape(ci, spherical, waves)
    NR = 17 + ci.L + 1 + 6 + 2
    return 8 * (_level_buffers(ci, spherical, waves, apart)[1] + NR * ((rb * Q) | 1))


def xd_apart(ci: ClassInfo, spherical: bool, waves: int = PACK_WAVES, rb: int = 0) -> bool:
    if not XD_APART:
        return False
    rb = rb or _k1_rb(ci, spherical)
    cap = 4 * _k1_waves_per_simd(ci, spherical) // waves
    return min(cap, LDS_BYTES // _lds_bytes(ci, spherical, waves, rb, True)) >= \
        min(cap, LDS_BYTES // _lds_bytes(ci, spherical, waves, rb, False))


def packed_lds_bytes(ci: ClassInfo, spherical: bool, waves: int = PACK_WAVES, rb: int = 0) -> int:
    rb = rb or _k1_rb(ci, spherical)
    return _lds_bytes(ci, spherical, waves, rb, xd_apart(ci, spherical, waves, rb))


def use_packed_k1(ci: ClassInfo, spherical: bool) -> bool:
    """Packing pays where a wave64 would leave many lanes idle, and a lane
    group wider than a wave needs it."""
    if wide_packed(ci, spherical):
        return packed_wg_per_cu(ci, spherical, packed_k1_waves(ci, spherical)) >= 1
    if ci.G > 64 or ci.G < 20:
        return False
    if (64 % ci.G) * 4 < 64:  # at most a quarter of the wave idles already
        return False
    if ci.Lk > 4:  # longer ket recurrences hold too many values for two waves per SIMD
        return False
    return packed_wg_per_cu(ci, spherical, packed_k1_waves(ci, spherical)) >= 2


def packed_wg_per_cu(ci: ClassInfo, spherical: bool, waves: int = PACK_WAVES, rb: int = 0) -> int:
    """Workgroups per compute unit: LDS-bound, at most two waves per SIMD
    (three for the kernels built for three)."""
    by_lds = LDS_BYTES // packed_lds_bytes(ci, spherical, waves, rb)
    return int(min(by_lds, 4 * _k1_waves_per_simd(ci, spherical) // waves))


def _lane_table(ci: ClassInfo, tag: str):
    """Constant table of the lane group (one entry per bra component e) and the
    lines that decode this lane's entry: e = (ex, ey, ez) and srcx/srcy/srcz, the
    lanes of e - 1_x, e - 1_y, e - 1_z in the same quartet (the lane itself where
    the component is 0).  Groups of up to 63 lanes pack 4-bit components and
    6-bit source fields into an int; up to 127 lanes (components up to 7), 3-bit
    components and 7-bit fields; wider groups, 4-bit components and 8-bit fields
    in a 64-bit entry."""
    lanes = ci.lanes
    G = len(lanes)
    lpos = {e: i for i, e in enumerate(lanes)}
    assert G <= 255
    if G >= 128:
        eb, sb, ty = 4, 8, "long long"
    elif G >= 64:
        eb, sb, ty = 3, 7, "int"
    else:
        eb, sb, ty = 4, 6, "int"
    assert max(max(e) for e in lanes) < (1 << eb)
    tab = []
    for e in lanes:
        d = [lpos[sub(e, ax)] if e[ax] > 0 else -1 for ax in range(3)]
        v = e[0] | (e[1] << eb) | (e[2] << 2 * eb)
        for ax in range(3):
            v |= (d[ax] + 1) << (3 * eb + ax * sb)
        tab.append(v)
    sfx = "LL" if ty == "long long" else ""
    decl = f"__constant__ {ty} k_{tag}_lane[{G}] = {{" + ", ".join(f"{v}{sfx}" for v in tab) + "};"
    em, sm = (1 << eb) - 1, (1 << sb) - 1
    cast = "(int)" if ty == "long long" else ""
    dec = [f"  const {ty} lt = k_{tag}_lane[sub];",
           f"  const int ex = {cast}(lt & {em}), ey = {cast}((lt >> {eb}) & {em}), ez = {cast}((lt >> {2 * eb}) & {em}),"
           f" es = ex + ey + ez;" if cast else
           f"  const int ex = lt & {em}, ey = (lt >> {eb}) & {em}, ez = (lt >> {2 * eb}) & {em}, es = ex + ey + ez;",
           "  const int qb = qi * G;"]
    for ax, nm in enumerate("xyz"):
        dec.append(f"  const int src{nm} = e{nm} > 0 ? qb + {cast}((lt >> {3 * eb + ax * sb}) & {sm}) - 1 : tid;")
    return decl, dec


# Level-buffer slots of the K4 = 1 kernels.  Lane t publishes its values at
# slot pi(t) and reads its coupling operands at pi(source lane).  A lane whose
# component along the read's axis is zero needs no operand (its factor e_i is
# zero); it reads a slot that another lane of its 16-lane group reads anyway,
# so the read adds no address.  pi is searched (fixed seed) so that the
# distinct addresses of every 16- and 32-lane group of a read and of the
# publishing write fall in distinct 8-byte banks modulo 16 and 32 -- the
# conflict-free pattern whether the LDS serves 16 lanes over 32 banks or 32
# lanes over 64 banks per cycle.  Measured on the (dd|dd) batch: 4% faster
# than identity slots with reads of the lane itself.
K1_SLOTS = True


def _source_lanes(lanes, NT: int):
    """Per axis, per lane t: the lane of e - 1_axis in t's quartet, or None where
    e_axis = 0 (spare lanes beyond the last quartet shadow e = 0)."""
    G = len(lanes)
    Q = NT // G
    lpos = {e: i for i, e in enumerate(lanes)}
    out = []
    for ax in range(3):
        col = []
        for t in range(NT):
            qi, sb = divmod(t, G)
            if qi >= Q:
                qi, sb = 0, 0
            e = lanes[sb]
            col.append(qi * G + lpos[sub(e, ax)] if e[ax] > 0 else None)
        out.append(col)
    return out


def slot_layout(ci: ClassInfo, NT: int):
    """(pi, reads): pi[t] is lane t's slot, reads[ax][t] the slot lane t reads
    along axis ax (see K1_SLOTS)."""
    return _slot_layout(tuple(ci.lanes), NT)


@functools.lru_cache(maxsize=None)
def _slot_layout(lanes, NT: int, iters: int = 20000, seed: int = 1):
    import random
    import numpy as np
    srcs = _source_lanes(lanes, NT)
    red = []
    for col in srcs:
        r = list(col)
        for t in range(NT):
            if r[t] is None:
                g0 = t - t % 16
                cand = [col[u] for u in range(g0, g0 + 16) if col[u] is not None]
                r[t] = min(cand, key=lambda v: abs(v - t)) if cand else g0
        red.append(r)
    # every access group: the distinct source lanes it touches, per bank modulus
    groups = []
    for width, mod in ((16, 16), (32, 32)):
        for col in red + [list(range(NT))]:
            for g0 in range(0, NT, width):
                groups.append((sorted(set(col[g0:g0 + width])), mod))
    ng = len(groups)
    L = max(len(g) for g, _ in groups)
    idx = np.full((ng, L), NT, dtype=np.int64)
    mods = np.array([m for _, m in groups], dtype=np.int64)
    for i, (g, _) in enumerate(groups):
        idx[i, :len(g)] = g

    def cost(pi):
        piv = np.append(pi, -1)[idx]  # padding maps to -1: a bank of its own
        b = np.where(piv < 0, 64, piv % mods[:, None])
        cnt = np.zeros((ng, 65), dtype=np.int64)
        np.add.at(cnt, (np.repeat(np.arange(ng), L), b.ravel()), 1)
        cnt[:, 64] = 0
        return int(cnt.max(axis=1).sum())
    rng = random.Random(seed)
    pi = np.arange(NT)
    cur = cost(pi)
    best_possible = ng
    for _ in range(iters):
        if cur == best_possible:
            break
        i, j = rng.randrange(NT), rng.randrange(NT)
        pi[i], pi[j] = pi[j], pi[i]
        c = cost(pi)
        if c <= cur:
            cur = c
        else:
            pi[i], pi[j] = pi[j], pi[i]
    pi = [int(v) for v in pi]
    return pi, [[pi[r] for r in col] for col in red]


SPLIT_BRA_HRR = True
# the bra HRR of the K4 = 1 kernels reads its whole exchange column up front
BRA_PRELOAD = True
# each ket level computes the lane's own terms before the barrier
K1_OWN_TERMS_FIRST = True


def bra_hrr_parts(ci: ClassInfo, spherical: bool, waves: int, Q: int, contracted: bool = False) -> int:
    """Waves that share the bra HRR phase.  It runs on (quartet, ket component)
    items, Q x (ket components) of them: for a lane group wider than a wave with
    a short ket that is a handful of lanes of the workgroup (3 of 192 for
    (gg|ps)).  When every item fits one wave, each wave instead takes every item
    and a 1/waves share of the bra outputs (the values those outputs need are
    recomputed per wave).  Measured against one item per lane: K4 = 1 kernels
    of (ff| 1.08-1.32x, (gf| 1.14-1.32x, (gg| 1.20-2.06x faster, (gd| even;
    contracted kernels even to 1.18x faster for 84- and 120-lane bras, but
    7-22% slower for (gg|, which keep one item per lane."""
    if not SPLIT_BRA_HRR or ci.G <= 64 or waves < 2 or Q * ci.nket(spherical) > 64:
        return 1
    if contracted and ci.G > 127:
        return 1
    return waves


def _emit_bra_hrr_split(ci, spherical, o, ind, P, slot_expr, setup, src_of):
    """Bra HRR and transform with the outputs split over the P waves (see
    bra_hrr_parts): wave w computes outputs [w nb / P, (w + 1) nb / P) of every
    item."""
    from .emit import _emit_hrr_scheduled
    nb = ci.nbra_out(spherical)
    o.append(f"{ind}{{  // bra HRR split by output over the waves: all items fit one wave")
    o.append(f"{ind}  const int part = __builtin_amdgcn_readfirstlane(tid >> 6), t = tid & 63;")
    o.append(f"{ind}  const int q2 = t / NK, kap = t - q2 * NK;")
    o.append(f"{ind}  const int slot = {slot_expr};")
    o.append(f"{ind}  if (t < Q * NK && slot < a.nq) {{")
    for l in setup:
        o.append(f"{ind}    {l}")
    o.append(f"{ind}    switch (part) {{")
    for p in range(P):
        lo, hi = p * nb // P, (p + 1) * nb // P
        o.append(f"{ind}    case {p}: {{")
        _emit_hrr_scheduled(ci.la, ci.lb, src_of, "AB", spherical,
                            lambda kk, x: f"eri_out_merged(&dst[{kk} * NK], {x});", o, ind + "      ", "z",
                            outputs=range(lo, hi))
        o.append(f"{ind}    }} break;")
    o.append(f"{ind}    default: break;")
    o.append(f"{ind}    }}")
    o.append(f"{ind}  }}")
    o.append(f"{ind}}}")


def emit_packed_k1(ci: ClassInfo, spherical: bool, waves: int = 0, rb: int = 0, wg_per_cu: int = 0,
                   min_waves: int = 0):
    """K4 = 1 kernel, Q quartets per workgroup of `waves` waves."""
    waves = waves or packed_k1_waves(ci, spherical)
    min_waves = min_waves or packed_k1_min_waves(ci, spherical)
    rb = rb or _k1_rb(ci, spherical)
    from .emit import Names, _stage1, _stage1_selectors, _emit_hrr_scheduled, _fmt, AX
    kv = build_ket_vrr(ci.lc, ci.Lk)
    names = Names("V", kv, ci.Lk)
    G = ci.G
    W, Q, NT = packed_shape(ci, spherical, waves)
    if not wg_per_cu:
        wg_per_cu = packed_wg_per_cu(ci, spherical, waves, rb)
    NK = ci.nket(spherical)
    NEB = ci.n_ebra
    EOFF = ci.e_bra_offset
    BLK = ci.nout(spherical)
    L = ci.L
    cid = class_id(ci.la, ci.lb, ci.lc, ci.ld)
    tag = f"c{cid}_{'s' if spherical else 'c'}_k1"
    lane_decl, lane_dec = _lane_table(ci, tag)
    if K1_SLOTS:
        pi, rd = slot_layout(ci, NT)
        assert NT <= 256
        tab = [pi[t] | (rd[0][t] << 8) | (rd[1][t] << 16) | (rd[2][t] << 24) for t in range(NT)]
        lane_decl += (f"\n__constant__ unsigned k_{tag}_slot[{NT}] = {{" +
                      ", ".join(f"{v}u" for v in tab) + "};")
        lane_dec = [ln for ln in lane_dec if not ln.lstrip().startswith("const int src")]
        lane_dec.append(f"  const unsigned slt = k_{tag}_slot[tid];")
        lane_dec.append("  const int myslot = (int)(slt & 255u), srcx = (int)((slt >> 8) & 255u),"
                        " srcy = (int)((slt >> 16) & 255u), srcz = (int)(slt >> 24);")
    me = "myslot" if K1_SLOTS else "tid"
    lv = _levels(kv)
    levels = sorted(lv)
    NC = max((len(v) for v in lv.values()), default=0)
    fields = ["PAx", "PAy", "PAz", "WPx", "WPy", "WPz", "QCx", "QCy", "QCz", "WQx", "WQy", "WQz",
              "i2z", "i2e", "roz", "roe", "i2ze"] + [f"F{m}" for m in range(L + 1)] + \
             ["CDx", "CDy", "CDz", "ABx", "ABy", "ABz"]
    NR = len(fields) + 2  # then two constant rows, 1.0 and 0.0, for the bra-path selectors
    RB = rb
    NRL = RB * Q
    assert NRL <= NT
    NX = Q * NEB * NK + NK  # exchange rows, then a junk row
    apart = xd_apart(ci, spherical, waves, rb)
    bufs, NU = _level_buffers(ci, spherical, waves, apart)
    assert NU >= NX
    o = []
    o.append("namespace {")
    o.append(lane_decl)
    o.append("}  // namespace")
    o.append(f"// {Q} quartets per workgroup of {NT} lanes ({Q * G} busy); ket coupling through LDS, level by level")
    lb = f"{NT}, {min_waves}" if min_waves else f"{NT}"
    o.append(f"__global__ void __launch_bounds__({lb}) eri_kernel_{tag}(EriClassArgs a)")
    o.append("{")
    o.append(f"  constexpr int G = {G}, Q = {Q}, NT = {NT}, NK = {NK}, NEB = {NEB}, BLK = {BLK};")
    o.append(f"  constexpr int RB = {RB}, NRL = {NRL}, NC = {max(NC, 1)};")
    # odd field stride: lanes reading different fields of one record hit different banks
    o.append(f"  constexpr int RS = {NRL | 1};")
    o.append(f"  // level buffers (two, alternating) during the recurrence; exchange afterwards")
    o.append(f"  __shared__ double xu[{NU}];")
    o.append(f"  __shared__ double rec[{NR} * RS];  // field-major quartet records of one batch")
    o.append("  const int tid = threadIdx.x;")
    o.append("  int qi = tid / G, sub = tid - qi * G;")
    o.append("  const bool real = qi < Q;")
    o.append("  if (!real) { qi = 0; sub = 0; }  // spare lanes shadow e = (0,0,0) of the first quartet")
    o += lane_dec
    o.append("  (void)srcx; (void)srcy; (void)srcz; (void)es;")
    o.append("  const int ngroups = (a.nq + Q - 1) / Q;")
    o.append(f"  if (tid < NRL) {{ rec[{NR - 2} * RS + tid] = 1.0; rec[{NR - 1} * RS + tid] = 0.0; }}")
    k1c = "all" if _k1_three(ci, spherical) else None
    _stage1_selectors(ci, o, "RS", NR - 2, NR - 1, compact=k1c)
    o.append(f"  double* xd = xu + ((real && es >= {ci.la}) ? (qi * NEB + (sub - {EOFF})) * NK : Q * NEB * NK);")
    o.append("  int it = 0;")
    o.append("  for (int g = blockIdx.x; g < ngroups; g += (int)gridDim.x, ++it) {")
    o.append("    const int bslot = it % RB;")
    o.append("    if (bslot == 0) {")
    o.append("      if (tid < NRL) {")
    o.append("        const int k = tid / Q, gk = g + k * (int)gridDim.x;")
    o.append("        int q = gk * Q + (tid - k * Q);")
    o.append("        if (gk >= ngroups || q >= a.nq) q = a.nq - 1;  // past the end: a valid record, never stored")
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
    # the three-wave kernels take exp(-T) from the table: exp()'s constants
    # would be held in registers across the loop and spill
    o.append(f"        eri_boys<{L}{', true' if _k1_three(ci, spherical) else ''}>(gq.T, gq.pref, a.boys, F);")
    vals = ["P.PA[0]", "P.PA[1]", "P.PA[2]", "gq.WP[0]", "gq.WP[1]", "gq.WP[2]", "K.PA[0]", "K.PA[1]", "K.PA[2]",
            "gq.WQ[0]", "gq.WQ[1]", "gq.WQ[2]", "0.5 * P.izeta", "0.5 * K.izeta", "gq.roz", "gq.roe", "gq.i2ze"]
    vals += [f"F[{m}]" for m in range(L + 1)]
    vals += ["Cx - a.cen[3 * pk.y]", "Cy - a.cen[3 * pk.y + 1]", "Cz - a.cen[3 * pk.y + 2]",
             "Ax - a.cen[3 * pb.y]", "Ay - a.cen[3 * pb.y + 1]", "Az - a.cen[3 * pb.y + 2]"]
    assert len(vals) == NR - 2
    o.append("        double* r = rec + tid;")
    for fi, v in enumerate(vals):
        o.append(f"        r[{fi} * RS] = {v};")
    o.append("      }")
    o.append("      __syncthreads();")
    o.append("    }")
    o.append("    const double* r = rec + bslot * Q + qi;")
    for fi, nm in enumerate(fields):
        if nm.startswith("F") or fi < 6 or nm.startswith("AB"):
            continue
        o.append(f"    const double {nm} = r[{fi} * RS];")
    o.append(f"    double F[{L + 1}];")
    for m in range(L + 1):
        o.append(f"    F[{m}] = r[{fields.index('F0') + m} * RS];")
    o.append("    (void)CDx; (void)CDy; (void)CDz;")
    o.append("    const double ehx = ex * i2ze, ehy = ey * i2ze, ehz = ez * i2ze;")
    o.append("    (void)QCx; (void)QCy; (void)QCz; (void)WQx; (void)WQy; (void)WQz; (void)i2z; (void)i2e;")
    o.append("    (void)roz; (void)roe; (void)ehx; (void)ehy; (void)ehz;")
    _stage1(ci, kv.base_m, o, "    ", rsel="r", compact=k1c)
    for li, k in enumerate(levels):
        buf = bufs[li]
        o.append(f"    // ket level {k}: publish level {k - 1} values read across lanes")
        for j, key in enumerate(lv[k]):
            o.append(f"    xu[{buf + j * NT} + {me}] = {names.ket(key)};")
        # the lane's own terms of every node first: they fill the wait for the
        # other waves at the barrier; only the coupling term follows the reads
        for n in kv.nodes:
            if sum(n.f) != k or not K1_OWN_TERMS_FIRST:
                continue
            a_ = AX[n.axis]
            expr = f"QC{a_} * {names.ket(n.a0)} + WQ{a_} * {names.ket(n.a1)}"
            if n.b0 is not None:
                expr += f" + {_fmt(n.fi_minus_1)} * i2e * ({names.ket(n.b0)} - roe * {names.ket(n.b1)})"
            o.append(f"    const double {names.ket((n.f, n.m))}p = {expr};")
        o.append("    __syncthreads();")
        reads = {}
        for n in kv.nodes:
            if sum(n.f) != k:
                continue
            rk = (lv[k].index(n.a1), n.axis)
            if rk not in reads:
                reads[rk] = f"xr{k}_{len(reads)}"
                o.append(f"    const double {reads[rk]} = xu[{buf + rk[0] * NT} + src{AX[n.axis]}];")
        if li == len(levels) - 1 and not apart:
            o.append("    __syncthreads();  // every level buffer read: the exchange may overwrite them")
        for n in kv.nodes:
            if sum(n.f) != k:
                continue
            a_ = AX[n.axis]
            own = f"{names.ket((n.f, n.m))}p"
            if not K1_OWN_TERMS_FIRST:
                own = f"QC{a_} * {names.ket(n.a0)} + WQ{a_} * {names.ket(n.a1)}"
                if n.b0 is not None:
                    own += f" + {_fmt(n.fi_minus_1)} * i2e * ({names.ket(n.b0)} - roe * {names.ket(n.b1)})"
            o.append(f"    const double {names.ket((n.f, n.m))} = {own}"
                     f" + eh{a_} * {reads[(lv[k].index(n.a1), n.axis)]};")
    # ket HRR and transform per lane, straight into the exchange row of this lane's e
    _emit_hrr_scheduled(ci.lc, ci.ld, lambda f: names.ket((f, 0)), "CD", spherical,
                        lambda kk, x: f"xd[{kk}] = {x};", o, "    ", "y")
    o.append("    __syncthreads();")
    # bra HRR and transform: lanes own (quartet, ket component)
    ab0 = fields.index("ABx")
    ebra = [e for l in range(ci.la, ci.Lb + 1) for e in components(l)]
    epos = {e: i for i, e in enumerate(ebra)}
    P = bra_hrr_parts(ci, spherical, W, Q)
    if P > 1:
        _emit_bra_hrr_split(ci, spherical, o, "    ", P, "g * Q + q2", [
            "const double* r2 = rec + bslot * Q + q2;",
            f"const double ABx = r2[{ab0} * RS], ABy = r2[{ab0 + 1} * RS], ABz = r2[{ab0 + 2} * RS];",
            "(void)ABx; (void)ABy; (void)ABz;",
            "const double* src = xu + q2 * NEB * NK + kap;",
            "double* dst = a.out + (size_t)slot * BLK + kap;"], lambda e: f"src[{epos[e]} * NK]")
    else:
        o.append("    for (int t = tid; t < Q * NK; t += NT) {")
        o.append("      const int q2 = t / NK, kap = t - q2 * NK;")
        o.append("      const int slot = g * Q + q2;")
        o.append("      if (slot >= a.nq) continue;")
        o.append("      const double* r2 = rec + bslot * Q + q2;")
        o.append(f"      const double ABx = r2[{ab0} * RS], ABy = r2[{ab0 + 1} * RS], ABz = r2[{ab0 + 2} * RS];")
        o.append("      (void)ABx; (void)ABy; (void)ABz;")
        o.append("      const double* src = xu + q2 * NEB * NK + kap;")
        o.append("      double* dst = a.out + (size_t)slot * BLK + kap;")
        _emit_hrr_scheduled(ci.la, ci.lb, lambda e: f"src[{epos[e]} * NK]", "AB", spherical,
                            lambda kk, x: f"eri_out_merged(&dst[{kk} * NK], {x});", o, "      ", "z",
                            preload=BRA_PRELOAD)
        o.append("    }")
    o.append("    __syncthreads();  // exchange and records are rewritten next")
    o.append("  }")
    o.append("}")
    o.append("")
    o.append(f"void eri_launch_{tag}(const EriClassArgs& a, hipStream_t s)")
    o.append("{")
    o.append(f"  const int ngroups = (a.nq + {Q} - 1) / {Q};")
    o.append(f"  const int cap = (a.grid_cap / 8) * {wg_per_cu};  // grid_cap is 8 per compute unit")
    o.append("  const int nblk = ngroups < cap ? ngroups : cap;")
    o.append(f"  if (nblk > 0) hipLaunchKernelGGL(eri_kernel_{tag}, dim3(nblk), dim3({NT}), 0, s, a);")
    o.append("}")
    o.append("")
    return o


PACK_CH = 21  # primitive quartets per quartet set up together (one lane each)
# the contracted packed kernels share the K4 = 1 kernels' conflict-free level
# slots, own-terms-first levels and bra-HRR preload
CONTRACTED_SLOTS = True
CONTRACTED_OWN_FIRST = True
CONTRACTED_PRELOAD = True
CONTRACTED_MIN_WAVES = 2  # waves per SIMD the contracted kernels are bounded to


# Register form of the contracted kernels.  With loop-invariant selectors (two
# offsets and a lowering count per bra step) and the set-up lanes' pair records
# kept across the primitive loop, the contracted (dd|dd) kernel needs a few
# registers over the 256 of two waves per SIMD and spilled 52 B per lane.  For
# it the selectors are packed into one int per step and the set-up state is
# re-read at every chunk (250 registers, nothing spilled); measured on the
# 120-atom cluster that form is 1.5% slower for (dd|dd) and 2-10% slower for
# the classes that do not spill, which keep the plain form.
COMPACT_CONTRACTED = {(2, 2, 2, 2)}


def _compact(ci: ClassInfo) -> bool:
    return (ci.la, ci.lb, ci.lc, ci.ld) in COMPACT_CONTRACTED


def _chunk(Q, NT, ch=0):
    return max(1, min(ch or PACK_CH, NT // Q))


def packed_contracted_waves(ci: ClassInfo) -> int:
    """Waves per workgroup of the contracted kernel.  Measured on the 120-atom
    cluster's class blocks: 35-lane bras with kets up to l = 3 run 5-10% faster
    with four waves (seven quartets, 245 of 256 lanes busy) than with two (three
    quartets, 105 of 128); with an l = 4 ket the level buffers then leave room
    for one workgroup per compute unit only, and two waves stay faster.  Three
    waves measured slower throughout."""
    if ci.G > 64:
        return _wide_waves(ci)
    if ci.G == 35 and ci.Lk <= 3:
        return 4
    return PACK_WAVES


def packed_contracted_lds_bytes(ci: ClassInfo, spherical: bool, waves: int = 0, ch: int = 0) -> int:
    kv = build_ket_vrr(ci.lc, ci.Lk)
    W, Q, NT = packed_shape(ci, spherical, waves or packed_contracted_waves(ci))
    ch = _chunk(Q, NT, ch)
    NC = max((len(v) for v in _levels(kv).values()), default=0)
    NX = Q * ci.n_ebra * ci.nket(spherical) + ci.nket(spherical)
    NR = 17 + ci.L + 1 + 2
    return 8 * (max(2 * NC * NT, NX) + NR * ((ch * Q) | 1)) + 4 * Q


def packed_contracted_wg_per_cu(ci: ClassInfo, spherical: bool, waves: int = 0) -> int:
    waves = waves or packed_contracted_waves(ci)
    return int(min(LDS_BYTES // packed_contracted_lds_bytes(ci, spherical, waves), 8 // waves))


def use_packed_contracted(ci: ClassInfo, spherical: bool) -> bool:
    """Measured on the 30-atom cluster: packing pays for 35-lane bras always,
    and for 20- and 10-lane bras once there is a ket recurrence whose
    coupling reads move from ds_bpermute to the level buffers.  A 56-lane bra
    fills a wave almost as well with one quartet per wave, but the level
    buffers still beat ds_bpermute there: 10-16% on the 120-atom cluster's
    (fd|pp) .. (fd|fp) blocks."""
    if wide_packed(ci, spherical):
        return packed_contracted_wg_per_cu(ci, spherical) >= 1
    if ci.Lk > 4:
        return False
    if not (ci.G == 35 or (ci.G in (20, 10, 56) and ci.Lk >= 1)):
        return False
    return packed_contracted_wg_per_cu(ci, spherical) >= 2


def emit_packed_contracted(ci: ClassInfo, spherical: bool, waves: int = 0, ch: int = 0):
    """General (contracted) kernel, Q quartets per workgroup of `waves` waves.

    Algorithm 2 of "FusionRCG": the primitive quartets of each quartet are set
    up in chunks (one lane per primitive quartet: geometry and Boys values into
    an LDS record), then every lane runs the bra path and the level-by-level
    ket recurrence for each primitive quartet of the chunk and adds its targets
    [e0|f0] into accumulators; the horizontal recurrences and transforms run
    once per quartet on the contracted values.  Quartets of one workgroup may
    differ in contraction length: the loop runs to the longest, and lanes of a
    shorter quartet evaluate its last primitive quartet again with weight 0."""
    from .emit import Names, _stage1, _stage1_selectors, _emit_hrr_scheduled, _fmt, AX
    kv = build_ket_vrr(ci.lc, ci.Lk)
    names = Names("V", kv, ci.Lk)
    G = ci.G
    waves = waves or packed_contracted_waves(ci)
    W, Q, NT = packed_shape(ci, spherical, waves)
    NK = ci.nket(spherical)
    NEB = ci.n_ebra
    EOFF = ci.e_bra_offset
    BLK = ci.nout(spherical)
    L = ci.L
    cid = class_id(ci.la, ci.lb, ci.lc, ci.ld)
    tag = f"c{cid}_{'s' if spherical else 'c'}"
    lane_decl, lane_dec = _lane_table(ci, tag)
    if CONTRACTED_SLOTS:
        pi, rd = slot_layout(ci, NT)
        assert NT <= 256
        tab = [pi[t] | (rd[0][t] << 8) | (rd[1][t] << 16) | (rd[2][t] << 24) for t in range(NT)]
        lane_decl += (f"\n__constant__ unsigned k_{tag}_slot[{NT}] = {{" +
                      ", ".join(f"{v}u" for v in tab) + "};")
        lane_dec = [ln for ln in lane_dec if not ln.lstrip().startswith("const int src")]
        lane_dec.append(f"  const unsigned slt = k_{tag}_slot[tid];")
        lane_dec.append("  const int myslot = (int)(slt & 255u), srcx = (int)((slt >> 8) & 255u),"
                        " srcy = (int)((slt >> 16) & 255u), srcz = (int)(slt >> 24);")
    me = "myslot" if CONTRACTED_SLOTS else "tid"
    lv = _levels(kv)
    levels = sorted(lv)
    NC = max((len(v) for v in lv.values()), default=0)
    fields = ["PAx", "PAy", "PAz", "WPx", "WPy", "WPz", "QCx", "QCy", "QCz", "WQx", "WQy", "WQz",
              "i2z", "i2e", "roz", "roe", "i2ze"] + [f"F{m}" for m in range(L + 1)]
    NR = len(fields) + 2  # then two constant rows, 1.0 and 0.0, for the bra-path selectors
    CH = _chunk(Q, NT, ch)
    NRL = Q * CH
    assert NRL <= NT
    NX = Q * NEB * NK + NK
    NU = max(2 * NC * NT, NX)
    targets = kv.targets
    tpos = {f: t for t, (f, m) in enumerate(targets)}
    o = []
    o.append("namespace {")
    o.append(lane_decl)
    o.append("}  // namespace")
    o.append(f"// {Q} quartets per workgroup of {NT} lanes ({Q * G} busy); ket coupling through LDS, level by level")
    # at least two waves per SIMD: (dd|dd), (fp|dd) and (fp|fp) otherwise take a
    # few registers over 256 and run at one; capped, they spill a few values and
    # measured 20-30% faster
    o.append(f"__global__ void __launch_bounds__({NT}, {CONTRACTED_MIN_WAVES}) eri_kernel_{tag}(EriClassArgs a)")
    o.append("{")
    o.append(f"  constexpr int G = {G}, Q = {Q}, NT = {NT}, NK = {NK}, NEB = {NEB}, BLK = {BLK};")
    o.append(f"  constexpr int CH = {CH}, NRL = {NRL}, NC = {max(NC, 1)};")
    o.append(f"  constexpr int RS = {NRL | 1};  // odd field stride: selector reads of one record hit different banks")
    o.append(f"  __shared__ double xu[{NU}];  // level buffers (two, alternating), then the exchange")
    o.append(f"  __shared__ double rec[{NR} * RS];  // field-major primitive-quartet records of one chunk")
    o.append("  __shared__ int k4q[Q];")
    o.append("  const int tid = threadIdx.x;")
    o.append("  int qi = tid / G, sub = tid - qi * G;")
    o.append("  const bool real = qi < Q;")
    o.append("  if (!real) { qi = 0; sub = 0; }  // spare lanes shadow e = (0,0,0) of the first quartet")
    o += lane_dec
    o.append("  (void)srcx; (void)srcy; (void)srcz; (void)es;")
    o.append(f"  if (tid < NRL) {{ rec[{NR - 2} * RS + tid] = 1.0; rec[{NR - 1} * RS + tid] = 0.0; }}")
    _stage1_selectors(ci, o, "RS", NR - 2, NR - 1, compact="all" if _compact(ci) else None)
    o.append("  const int g = blockIdx.x;")
    o.append("  const int q0 = g * Q;")
    o.append("  // this lane's quartet (the spare lanes and a short last group repeat a valid one)")
    o.append("  const int qme = q0 + qi < a.nq ? q0 + qi : a.nq - 1;")
    o.append("  const int4 pbm = a.pair_info[a.qbra[qme]], pkm = a.pair_info[a.qket[qme]];")
    o.append("  const int K4 = pbm.w * pkm.w;")
    o.append("  if (real && sub == 0) k4q[qi] = K4;")
    o.append("  // the quartet whose primitive quartets this lane sets up")
    o.append("  const int qsi = tid / CH < Q ? tid / CH : Q - 1;")
    o.append("  const int qs = q0 + qsi < a.nq ? q0 + qsi : a.nq - 1;")
    if not _compact(ci):
        o.append("  const int4 pbs = a.pair_info[a.qbra[qs]], pks = a.pair_info[a.qket[qs]];")
        o.append("  const double ACx = a.cen[3 * pbs.x] - a.cen[3 * pks.x], ACy = a.cen[3 * pbs.x + 1] - a.cen[3 * pks.x + 1],"
                 " ACz = a.cen[3 * pbs.x + 2] - a.cen[3 * pks.x + 2];")
        o.append("  const int K4s = pbs.w * pks.w;")
    o.append("  __syncthreads();")
    o.append("  int K4max = k4q[0];")
    o.append("  for (int i = 1; i < Q; ++i) K4max = k4q[i] > K4max ? k4q[i] : K4max;")
    for t in range(len(targets)):
        o.append(f"  double acc{t} = 0.0;")
    o.append("  int lvl = 0;  // running ket-level count: parity selects the level buffer")
    o.append("  for (int c0 = 0; c0 < K4max; c0 += CH) {")
    o.append("    if (c0 > 0) __syncthreads();  // the previous chunk's records are consumed")
    o.append("    if (tid < NRL) {")
    if _compact(ci):
        o.append("      // pair records and centres re-read per chunk (cached): nothing of the set-up")
        o.append("      // stays live in registers across the primitive loop")
        o.append("      const int4 pbs = a.pair_info[a.qbra[qs]], pks = a.pair_info[a.qket[qs]];")
        o.append("      const double ACx = a.cen[3 * pbs.x] - a.cen[3 * pks.x], ACy = a.cen[3 * pbs.x + 1] - a.cen[3 * pks.x + 1],"
                 " ACz = a.cen[3 * pbs.x + 2] - a.cen[3 * pks.x + 2];")
        o.append("      const int K4s = pbs.w * pks.w;")
    o.append("      const int p = c0 + (tid - qsi * CH);")
    o.append("      const int t = p < K4s ? p : K4s - 1;")
    o.append("      const int ib = t / pks.w, ik = t - ib * pks.w;")
    o.append("      const EriPrimPair P = eri_load_pp(a.ppd, pbs.z + ib);")
    o.append("      const EriPrimPair K = eri_load_pp(a.ppd, pks.z + ik);")
    o.append("      EriQuartetGeom gq;")
    o.append("      eri_geom(P, K, ACx, ACy, ACz, gq);")
    o.append(f"      double F[{L + 1}];")
    o.append(f"      eri_boys<{L}>(gq.T, gq.pref, a.boys, F);")
    vals = ["P.PA[0]", "P.PA[1]", "P.PA[2]", "gq.WP[0]", "gq.WP[1]", "gq.WP[2]", "K.PA[0]", "K.PA[1]", "K.PA[2]",
            "gq.WQ[0]", "gq.WQ[1]", "gq.WQ[2]", "0.5 * P.izeta", "0.5 * K.izeta", "gq.roz", "gq.roe", "gq.i2ze"]
    vals += [f"F[{m}]" for m in range(L + 1)]
    assert len(vals) == NR - 2
    o.append("      double* r = rec + tid;")
    for fi, v in enumerate(vals):
        o.append(f"      r[{fi} * RS] = {v};")
    o.append("    }")
    o.append("    __syncthreads();")
    o.append("    const int n = K4max - c0 < CH ? K4max - c0 : CH;")
    def segments(jexpr, wexpr, off_of):
        """One primitive quartet's code in phases: prologue, bra path, and per
        ket level (publish, own terms, reads, final terms); off_of[k] is the
        first level-buffer array of its level-k values."""
        pro = [f"      const double* r = rec + qi * CH + {jexpr};",
               f"      const double wgt = {wexpr};  // quartets shorter than the longest"]
        for fi, nm in enumerate(fields):
            if nm.startswith("F") or fi < 6:
                continue
            pro.append(f"      const double {nm} = r[{fi} * RS];")
        pro.append(f"      double F[{L + 1}];")
        for m in range(L + 1):
            pro.append(f"      F[{m}] = r[{fields.index('F0') + m} * RS];")
        pro.append("      const double ehx = ex * i2ze, ehy = ey * i2ze, ehz = ez * i2ze;")
        pro.append("      (void)QCx; (void)QCy; (void)QCz; (void)WQx; (void)WQy; (void)WQz; (void)i2z; (void)i2e;")
        pro.append("      (void)roz; (void)roe; (void)ehx; (void)ehy; (void)ehz;")
        bra = []
        _stage1(ci, kv.base_m, bra, "      ", rsel="r", compact="all" if _compact(ci) else None)
        for t, tg in enumerate(targets):
            if sum(tg[0]) == 0:
                bra.append(f"      acc{t} += wgt * s1_{tg[1]};")
        lvs = []
        for k in levels:
            pub = [f"        xb[{(off_of[k] + j) * NT}] = {names.ket(key)};" for j, key in enumerate(lv[k])]
            own = []
            if CONTRACTED_OWN_FIRST:
                for n in kv.nodes:
                    if sum(n.f) != k:
                        continue
                    a_ = AX[n.axis]
                    expr = f"QC{a_} * {names.ket(n.a0)} + WQ{a_} * {names.ket(n.a1)}"
                    if n.b0 is not None:
                        expr += f" + {_fmt(n.fi_minus_1)} * i2e * ({names.ket(n.b0)} - roe * {names.ket(n.b1)})"
                    own.append(f"      const double {names.ket((n.f, n.m))}p = {expr};")
            rds, reads = [], {}
            for n in kv.nodes:
                if sum(n.f) != k:
                    continue
                rk = (lv[k].index(n.a1), n.axis)
                if rk not in reads:
                    reads[rk] = f"xr{k}_{len(reads)}"
                    rds.append(f"      const double {reads[rk]} = xrb{k}[{(off_of[k] + rk[0]) * NT} + src{AX[n.axis]}];")
            fin = []
            for n in kv.nodes:
                if sum(n.f) != k:
                    continue
                a_ = AX[n.axis]
                if CONTRACTED_OWN_FIRST:
                    expr = f"{names.ket((n.f, n.m))}p"
                else:
                    expr = f"QC{a_} * {names.ket(n.a0)} + WQ{a_} * {names.ket(n.a1)}"
                    if n.b0 is not None:
                        expr += f" + {_fmt(n.fi_minus_1)} * i2e * ({names.ket(n.b0)} - roe * {names.ket(n.b1)})"
                expr += f" + eh{a_} * {reads[(lv[k].index(n.a1), n.axis)]}"
                fin.append(f"      const double {names.ket((n.f, n.m))} = {expr};")
                if n.m == 0 and n.f in tpos:
                    fin.append(f"      acc{tpos[n.f]} += wgt * {names.ket((n.f, n.m))};")
            lvs.append((pub, own, rds, fin))
        return pro, bra, lvs

    o.append("    for (int j = 0; j < n; ++j) {")
    pro, bra, lvs = segments("j", "c0 + j < K4 ? 1.0 : 0.0", {k: 0 for k in levels})
    o += pro + bra
    for li, k in enumerate(levels):
        pub, own, rds, fin = lvs[li]
        o.append(f"      // ket level {k}: publish level {k - 1} values read across lanes")
        o.append(f"      {{ double* xb = xu + (lvl & 1) * (NC * NT) + {me};")
        o += pub
        o.append("      }")
        o += own
        o.append("      __syncthreads();")
        o.append(f"      const double* xrb{k} = xu + (lvl & 1) * (NC * NT);")
        o.append("      ++lvl;")
        o += rds + fin
    o.append("    }")
    o.append("  }")
    o.append("  __syncthreads();  // level buffers and records read: the exchange may overwrite them")
    # ket HRR and transform per lane on the contracted values, into the exchange
    o.append("  const double CDx = a.cen[3 * pkm.x] - a.cen[3 * pkm.y], CDy = a.cen[3 * pkm.x + 1] - a.cen[3 * pkm.y + 1],"
             " CDz = a.cen[3 * pkm.x + 2] - a.cen[3 * pkm.y + 2];")
    o.append("  (void)CDx; (void)CDy; (void)CDz;")
    o.append(f"  double* xd = xu + ((real && es >= {ci.la}) ? (qi * NEB + (sub - {EOFF})) * NK : Q * NEB * NK);")
    _emit_hrr_scheduled(ci.lc, ci.ld, lambda f: f"acc{tpos[f]}", "CD", spherical,
                        lambda kk, x: f"xd[{kk}] = {x};", o, "  ", "y")
    o.append("  __syncthreads();")
    ebra = [e for l in range(ci.la, ci.Lb + 1) for e in components(l)]
    epos = {e: i for i, e in enumerate(ebra)}
    P = bra_hrr_parts(ci, spherical, W, Q, contracted=True)
    if P > 1:
        _emit_bra_hrr_split(ci, spherical, o, "  ", P, "q0 + q2", [
            "const int4 pb2 = a.pair_info[a.qbra[slot]];",
            "const double ABx = a.cen[3 * pb2.x] - a.cen[3 * pb2.y], ABy = a.cen[3 * pb2.x + 1] - a.cen[3 * pb2.y + 1],"
            " ABz = a.cen[3 * pb2.x + 2] - a.cen[3 * pb2.y + 2];",
            "(void)ABx; (void)ABy; (void)ABz;",
            "const double* src = xu + q2 * NEB * NK + kap;",
            "double* dst = a.out + (size_t)slot * BLK + kap;"], lambda e: f"src[{epos[e]} * NK]")
    else:
        o.append("  for (int t = tid; t < Q * NK; t += NT) {")
        o.append("    const int q2 = t / NK, kap = t - q2 * NK;")
        o.append("    const int slot = q0 + q2;")
        o.append("    if (slot >= a.nq) continue;")
        o.append("    const int4 pb2 = a.pair_info[a.qbra[slot]];")
        o.append("    const double ABx = a.cen[3 * pb2.x] - a.cen[3 * pb2.y], ABy = a.cen[3 * pb2.x + 1] - a.cen[3 * pb2.y + 1],"
                 " ABz = a.cen[3 * pb2.x + 2] - a.cen[3 * pb2.y + 2];")
        o.append("    (void)ABx; (void)ABy; (void)ABz;")
        o.append("    const double* src = xu + q2 * NEB * NK + kap;")
        o.append("    double* dst = a.out + (size_t)slot * BLK + kap;")
        _emit_hrr_scheduled(ci.la, ci.lb, lambda e: f"src[{epos[e]} * NK]", "AB", spherical,
                            lambda kk, x: f"eri_out_merged(&dst[{kk} * NK], {x});", o, "    ", "z",
                            preload=CONTRACTED_PRELOAD)
        o.append("  }")
    o.append("}")
    o.append("")
    o.append(f"void eri_launch_{tag}(const EriClassArgs& a, hipStream_t s)")
    o.append("{")
    o.append(f"  const int ngroups = (a.nq + {Q} - 1) / {Q};  // one group per workgroup")
    o.append(f"  if (ngroups > 0) hipLaunchKernelGGL(eri_kernel_{tag}, dim3(ngroups), dim3({NT}), 0, s, a);")
    o.append("}")
    o.append("")
    return o
