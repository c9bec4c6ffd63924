"""CPU checks of the kernel generator (no GPU).

* the generator's spherical coefficients (recursion) against the oracle's
  (closed form) -- two independent derivations of Eq. (8)'s t^(l);
* a numpy emulation of the generated algorithm (lane-owns-e bra paths, ket
  vertical recurrence with the cross-lane coupling term, contraction, both
  horizontal phases and stepwise transforms) executed from the generator's
  own graphs, against the oracle, for every class up to (dd|dd) and a few
  higher ones;
* class enumeration and tier routing.
"""
import math
import os

import numpy as np
import pytest

import oracle
from electron_repulsion_integrals_amd.gen import cartesian as gc
from electron_repulsion_integrals_amd.gen import graph as gg
from workloads.configs import _pack


@pytest.mark.parametrize("l", range(7))
def test_generator_sph_matches_oracle(l):
    np.testing.assert_allclose(np.array(gc.sph_matrix(l)), oracle.sph_coeffs(l), atol=1e-13)


def test_class_enumeration():
    cls = gg.all_classes(4)
    assert len(cls) == 120
    ids = [gg.class_id(c.la, c.lb, c.lc, c.ld) for c in cls]
    assert sorted(ids) == list(range(120))


def _norm(l, exps, coefs):
    df = 1.0
    for t in range(2 * l - 1, 1, -2):
        df *= t
    c = np.array([cf * (2 * a / math.pi) ** 0.75 * (4 * a) ** (l / 2) / math.sqrt(df) for a, cf in zip(exps, coefs)])
    s = sum(c[i] * c[j] * (math.pi / (exps[i] + exps[j])) ** 1.5 * df / (2 * (exps[i] + exps[j])) ** l
            for i in range(len(c)) for j in range(len(c)))
    return c / math.sqrt(s)


def _boys(L, T):
    # reference values for the emulation only (the device uses its own table)
    return oracle.boys(L, T)


def emulate(ci, cen, exps, coefs, spherical):
    """Run the generated algorithm for one quartet, lane by lane, in numpy."""
    A, B, C, D = [np.asarray(x, dtype=float) for x in cen]
    ls = (ci.la, ci.lb, ci.lc, ci.ld)
    cn = [_norm(l, e, c) for l, e, c in zip(ls, exps, coefs)]
    lanes = ci.lanes
    lpos = {e: i for i, e in enumerate(lanes)}
    kv = gg.build_ket_vrr(ci.lc, ci.Lk)
    L = ci.L
    acc = {t: np.zeros(len(lanes)) for t in kv.targets}
    for ia, al in enumerate(exps[0]):
        for ib, be in enumerate(exps[1]):
            z = al + be
            P = (al * A + be * B) / z
            Kab = cn[0][ia] * cn[1][ib] * math.exp(-al * be / z * np.sum((A - B) ** 2)) / z
            for ic, ga in enumerate(exps[2]):
                for id_, de in enumerate(exps[3]):
                    e_ = ga + de
                    Q = (ga * C + de * D) / e_
                    Kcd = cn[2][ic] * cn[3][id_] * math.exp(-ga * de / e_ * np.sum((C - D) ** 2)) / e_
                    ize = 1 / (z + e_)
                    rho = z * e_ * ize
                    W = (z * P + e_ * Q) * ize
                    PA, WP, QC, WQ = P - A, W - P, Q - C, W - Q
                    T = rho * np.sum((P - Q) ** 2)
                    pref = 2 * math.pi ** 2.5 * Kab * Kcd * math.sqrt(ize)
                    F = pref * _boys(L, T)
                    i2z, roz, i2e, roe, i2ze = 0.5 / z, e_ * ize, 0.5 / e_, z * ize, 0.5 * ize
                    # bra phase per lane: [e0|00]^(m)
                    s1 = np.zeros((len(lanes), L + 1))
                    for li, e in enumerate(lanes):
                        cur = F.copy()
                        prev = np.zeros(L + 1)
                        steps = [0] * e[0] + [1] * e[1] + [2] * e[2]
                        cnt = [0, 0, 0]
                        for s, ax in enumerate(steps, start=1):
                            n = cnt[ax]
                            new = np.zeros(L + 1)
                            for m in range(L - s + 1):
                                new[m] = PA[ax] * cur[m] + WP[ax] * cur[m + 1] + n * i2z * (prev[m] - roz * prev[m + 1])
                            prev, cur = cur, new
                            cnt[ax] += 1
                        s1[li] = cur
                    # ket phase: V[(f, m)] is a vector over lanes
                    V = {((0, 0, 0), m): s1[:, m].copy() for m in range(kv.base_m + 1)}
                    for nd in kv.nodes:
                        ax = nd.axis
                        v = QC[ax] * V[nd.a0] + WQ[ax] * V[nd.a1]
                        if nd.b0 is not None:
                            v = v + nd.fi_minus_1 * i2e * (V[nd.b0] - roe * V[nd.b1])
                        remote = np.array([V[nd.a1][lpos[gc.sub(e, ax)]] if e[ax] > 0 else 0.0 for e in lanes])
                        eh = np.array([e[ax] for e in lanes]) * i2ze
                        V[(nd.f, nd.m)] = v + eh * remote
                    for t in kv.targets:
                        acc[t] += V[t]
    # ket HRR per lane (lane = e), then transform
    hn, base = gg.build_hrr(ci.lc, ci.ld)
    CD = C - D
    H = {(f, (0, 0, 0)): acc[(f, 0)] for f in base}
    for nd in hn:
        H[(nd.x, nd.y)] = H[nd.p_hi] + CD[nd.axis] * H[nd.p_lo]
    cs, ds = gc.components(ci.lc), gc.components(ci.ld)
    Y = np.array([[H[(c, d)] for d in ds] for c in cs])  # [nc, nd, lanes]
    if spherical:
        Y = np.einsum("sd,cdl->csl", np.array(gc.sph_matrix(ci.ld)), Y)
        Y = np.einsum("rc,csl->rsl", np.array(gc.sph_matrix(ci.lc)), Y)
    Y = Y.reshape(-1, len(lanes))  # [kappa, lanes]
    # bra HRR per kappa
    hb, baseb = gg.build_hrr(ci.la, ci.lb)
    AB = A - B
    G = {(e, (0, 0, 0)): Y[:, lpos[e]] for e in baseb}
    for nd in hb:
        G[(nd.x, nd.y)] = G[nd.p_hi] + AB[nd.axis] * G[nd.p_lo]
    as_, bs = gc.components(ci.la), gc.components(ci.lb)
    Z = np.array([[G[(a, b)] for b in bs] for a in as_])  # [na, nb, kappa]
    if spherical:
        Z = np.einsum("sb,abk->ask", np.array(gc.sph_matrix(ci.lb)), Z)
        Z = np.einsum("ra,ask->rsk", np.array(gc.sph_matrix(ci.la)), Z)
    f = gc.nsph if spherical else gc.ncart
    return Z.reshape(f(ci.la), f(ci.lb), f(ci.lc), f(ci.ld))


CLASSES = [(0, 0, 0, 0), (1, 0, 0, 0), (1, 0, 1, 0), (1, 1, 0, 0), (1, 1, 1, 0), (1, 1, 1, 1), (2, 0, 0, 0),
           (2, 0, 1, 1), (2, 1, 2, 0), (2, 2, 1, 0), (2, 2, 2, 1), (2, 2, 2, 2), (3, 1, 2, 1), (3, 3, 1, 0), (4, 0, 2, 2)]


@pytest.mark.parametrize("ls", CLASSES)
@pytest.mark.parametrize("spherical", [False, True])
def test_emulated_algorithm_matches_oracle(ls, spherical):
    ci = gg.ClassInfo(*ls)
    rng = np.random.default_rng(sum(ls) * 13 + spherical)
    cen = [rng.uniform(0, 4, 3) for _ in range(4)]
    K = [2, 1, 2, 1]
    exps = [list(np.exp(rng.uniform(np.log(0.2), np.log(8.0), k))) for k in K]
    coefs = [list(rng.uniform(0.2, 1.0, k)) for k in K]
    got = emulate(ci, cen, exps, coefs, spherical)
    sh = _pack(cen, list(ls), K, [np.array(e) for e in exps], [np.array(c) for c in coefs])
    ref = oracle.eri_block(sh, [0, 1, 2, 3], spherical)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-13 * max(1.0, np.abs(ref).max()))


def test_tier_routing():
    from electron_repulsion_integrals_amd.gen.emit import tier_of
    for c in gg.all_classes(2):
        assert tier_of(c) == "V", (c.la, c.lb, c.lc, c.ld)
    # an l = 6 ket of an 84-lane bra runs packed for spherical output only
    assert tier_of(gg.ClassInfo(3, 3, 3, 3), True) == "V" and tier_of(gg.ClassInfo(3, 3, 3, 3), False) == "M"
    assert tier_of(gg.ClassInfo(4, 4, 4, 4)) == "M"


def test_packed_k1_routing_and_shapes():
    """Classes whose bra spans 35 lanes, and 84- and 120-lane bras with a short ket, run
    the uncontracted kernel with several quartets per workgroup; the lane
    layout, record batch and LDS plan fit."""
    from electron_repulsion_integrals_amd.gen import packed as P
    from electron_repulsion_integrals_amd.gen.emit import emit_register_tier
    used = []
    for c in gg.all_classes(4):
        for sph in (False, True):
            if not P.use_packed_k1(c, sph):
                continue
            used.append((c.la, c.lb, c.lc, c.ld))
            W, Q, NT = P.packed_shape(c, sph, P.packed_k1_waves(c, sph))
            three = (c.la, c.lb, c.lc, c.ld, sph) in P.K1_THREE_WAVES
            assert c.G in (35, 84, 120, 165) and Q * c.G <= NT and P._k1_rb(c, sph) * Q <= NT
            assert W == (3 if three else {84: 4, 165: 3}.get(c.G, 2))
            wg = P.packed_wg_per_cu(c, sph, W)
            assert 1 <= wg and P.packed_lds_bytes(c, sph, W) * wg <= P.LDS_BYTES
            # two waves per SIMD at most, three for the kernels built for three
            assert wg * W <= 4 * (3 if three else 2)
            src = emit_register_tier(c, sph)
            if "lane tier" not in src.splitlines()[0]:
                mw = P.packed_k1_min_waves(c, sph)
                lb = f"{NT}, {mw}" if mw else f"{NT}"
                assert f"__launch_bounds__({lb}) eri_kernel_" in src and "_k1(" in src and "xu[" in src
    assert (2, 2, 2, 2) in used and (3, 1, 2, 2) in used and (3, 3, 2, 1) in used
    assert (4, 3, 4, 1) in used and (4, 3, 3, 3) not in used
    assert P.packed_k1_min_waves(gg.ClassInfo(3, 3, 2, 2)) == 2 and P.packed_k1_min_waves(gg.ClassInfo(4, 3, 1, 0)) == 0
    # spherical (dd|dd): three waves per SIMD, four three-wave workgroups per compute unit
    dd = gg.ClassInfo(2, 2, 2, 2)
    assert P.packed_k1_waves(dd, True) == 3 and P.packed_k1_min_waves(dd, True) == 3
    assert P.packed_wg_per_cu(dd, True, 3) == 4 and P.packed_shape(dd, True, 3) == (3, 5, 192)
    assert P.packed_k1_min_waves(dd, False) == 0
    assert all(sum(u[:2]) in (4, 6, 7, 8) and sum(u[2:]) <= {4: 4, 6: 6, 7: 5, 8: 4}[sum(u[:2])] for u in used)
    assert (4, 4, 2, 2) in used and (4, 4, 3, 2) not in used



def test_packed_contracted_routing_and_shapes():
    """Contracted classes whose bra spans 20, 35, 56, 84 or 120 lanes (with a ket
    recurrence, outside the one-quartet-per-lane tier) run several quartets per multi-wave workgroup: the quartets,
    the set-up chunk and the LDS plan fit, and the emitted kernel has the
    planned shape."""
    from electron_repulsion_integrals_amd.gen import packed as P
    from electron_repulsion_integrals_amd.gen.emit import emit_register_tier, tier_of
    from electron_repulsion_integrals_amd.gen.lane import use_lane_tier
    used = {}
    for c in gg.all_classes(4):
        if use_lane_tier(c, True):
            continue
        for sph in (False, True):
            if tier_of(c, sph) != "V" or not P.use_packed_contracted(c, sph):
                continue
            W = P.packed_contracted_waves(c)
            _, Q, NT = P.packed_shape(c, sph, W)
            ch = P._chunk(Q, NT)
            assert Q >= 1 and Q * c.G <= NT and ch * Q <= NT
            assert 1 <= P.packed_contracted_wg_per_cu(c, sph) and \
                P.packed_contracted_lds_bytes(c, sph) * P.packed_contracted_wg_per_cu(c, sph) <= P.LDS_BYTES
            src = emit_register_tier(c, sph)
            assert f"__launch_bounds__({NT}, 2)" in src and f"dim3({NT})" in src
            used[(c.la, c.lb, c.lc, c.ld)] = (c.G, W, Q)
    assert used[(2, 2, 2, 1)] == (35, 4, 7) and used[(2, 2, 2, 2)] == (35, 2, 3)
    assert used[(3, 2, 2, 1)] == (56, 2, 2) and used[(2, 1, 2, 1)] == (20, 2, 6)
    assert used[(3, 3, 1, 0)] == (84, 4, 3) and used[(4, 2, 4, 0)] == (84, 4, 3) and used[(3, 3, 3, 2)] == (84, 4, 3)
    assert used[(3, 3, 3, 3)] == (84, 4, 3) and (3, 2, 3, 2) not in used
    assert used[(4, 3, 2, 1)] == (120, 2, 1) and (4, 3, 3, 3) not in used
    assert used[(4, 4, 1, 0)] == (165, 3, 1)
    assert all(v[0] in (10, 20, 35, 56, 84, 120, 165) for v in used.values())


def test_packed_lane_table_decodes():
    """The packed kernels' lane table (4-bit components and 6-bit source lanes
    below 64 lanes, 3-bit and 7-bit up to 127, 4-bit and 8-bit in 64-bit entries
    beyond) decodes to each lane's bra component and the lanes of its lower
    neighbours."""
    import re
    from electron_repulsion_integrals_amd.gen import packed as P
    from electron_repulsion_integrals_amd.gen.cartesian import sub
    for c in (gg.ClassInfo(2, 2, 1, 1), gg.ClassInfo(3, 2, 2, 1), gg.ClassInfo(3, 3, 1, 0), gg.ClassInfo(4, 3, 1, 0),
              gg.ClassInfo(4, 4, 1, 0)):
        decl, dec = P._lane_table(c, "t")
        assert ("long long" in decl) == (c.G >= 128)
        tab = [int(v.strip().rstrip("L")) for v in re.search(r"\{(.*)\}", decl).group(1).split(",")]
        text = "\n".join(dec)
        em = int(re.search(r"lt & (\d+)", text).group(1))
        shifts = [(int(a), int(b)) for a, b in re.findall(r">> (\d+)\) & (\d+)", text)]
        eb = shifts[0][0]
        src = shifts[2:5]
        lpos = {e: i for i, e in enumerate(c.lanes)}
        assert len(tab) == c.G and len(src) == 3
        for i, e in enumerate(c.lanes):
            v = tab[i]
            assert (v & em, (v >> eb) & em, (v >> 2 * eb) & em) == e
            for ax in range(3):
                want = lpos[sub(e, ax)] + 1 if e[ax] > 0 else 0
                assert (v >> src[ax][0]) & src[ax][1] == want


def test_split_bra_hrr_covers_outputs_once():
    """Lane groups wider than a wave with a short ket split the bra HRR over the
    waves: each wave's share defines every value it uses, and the shares
    together store each bra output exactly once."""
    import re
    from electron_repulsion_integrals_amd.gen import packed as P
    from electron_repulsion_integrals_amd.gen.emit import emit_register_tier
    for c, sph in ((gg.ClassInfo(3, 3, 1, 0), True), (gg.ClassInfo(4, 4, 1, 1), False), (gg.ClassInfo(4, 3, 2, 0), True)):
        src = emit_register_tier(c, sph)
        W, Q, NT = P.packed_shape(c, sph, P.packed_k1_waves(c, sph))
        assert P.bra_hrr_parts(c, sph, W, Q) == W > 1
        kernels = src.split("__global__")[1:]
        assert len(kernels) == 2
        # the contracted (gg| kernels keep one item per lane
        assert ("bra HRR split" in kernels[0]) == (c.G < 128) and "bra HRR split" in kernels[1]
        for kern in kernels:
            if "bra HRR split" not in kern:
                continue
            body = kern[kern.index("bra HRR split"):]
            cases = re.split(r"\n\s*case \d+: \{", body)[1:]
            assert len(cases) == W
            stored = []
            for cs in cases:
                defined = set()
                for line in cs[:cs.index("} break;")].splitlines():
                    m = re.match(r"\s*const double (z[bo]\d+) = (.*);", line)
                    used = re.findall(r"\bz[bo]\d+\b", m.group(2) if m else line)
                    assert all(u in defined for u in used), line
                    if m:
                        defined.add(m.group(1))
                    stored += [int(k) for k in re.findall(r"eri_out_merged\(&dst\[(\d+) \* NK\]", line)]
            assert sorted(stored) == list(range(c.nbra_out(sph)))
    # lane groups of one wave keep the one-item-per-lane loop
    c = gg.ClassInfo(2, 2, 2, 2)
    assert "bra HRR split" not in emit_register_tier(c, True)



def _apply_ops(ops, base_val, R):
    """Evaluate the generator's linear HRR/transform ops (emit._hrr_ops)."""
    val = dict(base_val)
    for key, terms in ops:
        tot = 0.0
        for c, src in terms:
            if c is None:
                w = 1.0
            elif c[:2] in ("AB", "CD"):
                w = R["xyz".index(c[2])]
            else:
                w = float(c)
            tot = tot + w * val[src]
        val[key] = tot
    return val


def emulate_lane_tier(ci, cen, exps, coefs, spherical):
    """The lane tier's graph (gen.lane.lane_vrr) and the generator's horizontal
    ops evaluated in numpy for one quartet, in the order the kernel uses."""
    from electron_repulsion_integrals_amd.gen import lane as LN
    from electron_repulsion_integrals_amd.gen.emit import _hrr_ops
    A, B, C, D = [np.asarray(x, dtype=float) for x in cen]
    ls = (ci.la, ci.lb, ci.lc, ci.ld)
    cn = [_norm(l, e, c) for l, e, c in zip(ls, exps, coefs)]
    nodes, targets, ebra, kv = LN.lane_vrr(ci)
    order = sorted((k for k, v in nodes.items() if v[0] != "F"), key=lambda k: (sum(k[0]) + sum(k[1]), -k[2]))
    acc = {t: 0.0 for t in targets}
    for ia, al in enumerate(exps[0]):
        for ib, be in enumerate(exps[1]):
            z = al + be
            P = (al * A + be * B) / z
            Kab = cn[0][ia] * cn[1][ib] * math.exp(-al * be / z * np.sum((A - B) ** 2)) / z
            for ic, ga in enumerate(exps[2]):
                for id_, de in enumerate(exps[3]):
                    e_ = ga + de
                    Q = (ga * C + de * D) / e_
                    Kcd = cn[2][ic] * cn[3][id_] * math.exp(-ga * de / e_ * np.sum((C - D) ** 2)) / e_
                    ize = 1 / (z + e_)
                    W = (z * P + e_ * Q) * ize
                    PA, WP, QC, WQ = P - A, W - P, Q - C, W - Q
                    T = z * e_ * ize * np.sum((P - Q) ** 2)
                    F = 2 * math.pi ** 2.5 * Kab * Kcd * math.sqrt(ize) * _boys(ci.L, T)
                    i2z, roz, i2e, roe, i2ze = 0.5 / z, e_ * ize, 0.5 / e_, z * ize, 0.5 * ize
                    V = {k: F[k[2]] for k, v in nodes.items() if v[0] == "F"}
                    for k in order:
                        kind, ax, dl = nodes[k]
                        e, f = k[0], k[1]
                        if kind == "b":
                            v = PA[ax] * V[dl[0]] + WP[ax] * V[dl[1]]
                            if e[ax] >= 2:
                                v += (e[ax] - 1) * i2z * (V[dl[2]] - roz * V[dl[3]])
                            if f[ax] > 0:
                                v += f[ax] * i2ze * V[dl[-1]]
                        else:
                            v = QC[ax] * V[dl[0]] + WQ[ax] * V[dl[1]]
                            if f[ax] >= 2:
                                v += (f[ax] - 1) * i2e * (V[dl[2]] - roe * V[dl[3]])
                            if e[ax] > 0:
                                v += e[ax] * i2ze * V[dl[-1]]
                        V[k] = v
                    for (e, f) in targets:
                        acc[(e, f)] += V[(e, f, 0)]
    kops, kbase, kouts = _hrr_ops(ci.lc, ci.ld, "CD", spherical)
    bops, bbase, bouts = _hrr_ops(ci.la, ci.lb, "AB", spherical)
    Y = {}
    for e in ebra:
        val = _apply_ops(kops, {("b", f): acc[(e, f)] for f in kbase}, C - D)
        for ki, ko in enumerate(kouts):
            Y[(e, ki)] = val[ko]
    out = np.zeros((len(bouts), len(kouts)))
    for ki in range(len(kouts)):
        val = _apply_ops(bops, {("b", e): Y[(e, ki)] for e in bbase}, A - B)
        for bi, bo in enumerate(bouts):
            out[bi, ki] = val[bo]
    f = gc.nsph if spherical else gc.ncart
    return out.reshape(f(ci.la), f(ci.lb), f(ci.lc), f(ci.ld))


@pytest.mark.parametrize("ls", [(1, 1, 1, 0), (2, 0, 2, 0), (2, 1, 1, 0), (3, 2, 0, 0), (4, 2, 0, 0)])
@pytest.mark.parametrize("spherical", [False, True])
def test_lane_tier_graph_matches_oracle(ls, spherical):
    """The one-quartet-per-lane graph and its horizontal ops reproduce the oracle."""
    from electron_repulsion_integrals_amd.gen import lane as LN
    ci = gg.ClassInfo(*ls)
    assert LN.use_lane_tier(ci, spherical)
    rng = np.random.default_rng(sum(ls) * 7 + spherical)
    cen = [rng.uniform(0, 4, 3) for _ in range(4)]
    K = [2, 1, 2, 2]
    exps = [list(np.exp(rng.uniform(np.log(0.2), np.log(8.0), k))) for k in K]
    coefs = [list(rng.uniform(0.2, 1.0, k)) for k in K]
    got = emulate_lane_tier(ci, cen, exps, coefs, spherical)
    sh = _pack(cen, list(ls), K, [np.array(e) for e in exps], [np.array(c) for c in coefs])
    ref = oracle.eri_block(sh, [0, 1, 2, 3], spherical)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-13 * max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("topology", ["alg1", "bra_first"])
@pytest.mark.parametrize("ls", [(1, 1, 1, 0), (2, 1, 1, 1), (3, 0, 2, 0)])
def test_lane_tier_topology_variants_match_oracle(ls, topology):
    """The ablation graphs (the printed axis-priority rule of Algorithm 1, and
    bra side first) are other valid graphs of Eq. (2): evaluated in numpy they
    reproduce the oracle, with bra nodes carrying the ket coupling term."""
    from electron_repulsion_integrals_amd.gen import variant, lane as LN
    ci = gg.ClassInfo(*ls)
    rng = np.random.default_rng(sum(ls) * 11 + len(topology))
    cen = [rng.uniform(0, 4, 3) for _ in range(4)]
    K = [2, 1, 1, 2]
    exps = [list(np.exp(rng.uniform(np.log(0.2), np.log(8.0), k))) for k in K]
    coefs = [list(rng.uniform(0.2, 1.0, k)) for k in K]
    prev = variant.set_variant(variant.Variant(name="t", topology=topology))
    try:
        nodes, _, _, _ = LN.lane_vrr(ci)
        assert any(k == "b" and sum(key[1]) > 0 for key, (k, _, _) in nodes.items())
        got = emulate_lane_tier(ci, cen, exps, coefs, True)
    finally:
        variant.set_variant(prev)
    sh = _pack(cen, list(ls), K, [np.array(e) for e in exps], [np.array(c) for c in coefs])
    ref = oracle.eri_block(sh, [0, 1, 2, 3], True)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-13 * max(1.0, np.abs(ref).max()))


def test_topological_order_variant_is_valid_and_plain():
    """The scheduler of the no-DSA variant returns a topological order of the same
    items (every operand before its consumer) without reordering for liveness; on
    a lane-tier graph its PeakLive is above the liveness scheduler's."""
    from electron_repulsion_integrals_amd.gen import variant, lane as LN
    ci = gg.ClassInfo(2, 1, 1, 1)
    nodes, targets, ebra, kv = LN.lane_vrr(ci)
    peaks = {}
    for sched in ("dsa", "topo"):
        prev = variant.set_variant(variant.Variant(name=sched, schedule=sched))
        try:
            _, _, _, _, order, base = LN._schedule(ci)
        finally:
            variant.set_variant(prev)
        seen = set(base)
        for k, ds, sink in order:
            assert all(d in seen for d in ds), k
            seen.add(k)
        assert len(order) == len(nodes) - len(base) + len(targets)
        peaks[sched] = gg.peak_live(order, None, base)
    assert peaks["topo"] > peaks["dsa"], peaks


def test_lane_tier_graph_is_the_counted_graph():
    """Per primitive quartet the lane tier evaluates exactly the recurrence nodes
    that the FLOP count of the roofline reports (graph.dag_flops)."""
    from electron_repulsion_integrals_amd.gen import lane as LN
    for ls in [(1, 1, 1, 0), (2, 1, 1, 0), (2, 0, 2, 0), (4, 2, 0, 0)]:
        ci = gg.ClassInfo(*ls)
        nodes, targets, ebra, kv = LN.lane_vrr(ci)
        flops = 0
        for (e, f, m), (kind, ax, dl) in nodes.items():
            if kind == "b":
                assert f == (0, 0, 0)
                flops += 3 + (4 if e[ax] >= 2 else 0)
            elif kind == "k":
                flops += 3 + (4 if f[ax] >= 2 else 0) + (2 if e[ax] > 0 else 0)
        per_prim, _ = gg.dag_flops(ci, True)
        other = 30 + 14 + 3 * ci.L + (ci.L + 1) + ci.n_ebra * len(kv.targets)
        assert flops == per_prim - other, ls


def test_two_phase_fp64_floor_bounds_the_emulated_algorithm():
    """On diffuse (gg|gg) and (ff|ff) quartets ~7 bohr apart the fp64 two-phase
    evaluation loses up to 1e-5 of the block maximum; the oracle's first-order
    floor (fp64 rounding of [e0|f0] through the unrolled HRR) bounds that loss."""
    from oracle import plan as oplan
    from workloads import make_config
    w = make_config(4, scale={"nquartets_f": 64, "nquartets_g": 16})
    sh = w.shells
    imap = oplan.explicit_plan(sh.l, sh.nprim, w.quartets)["index_map"]
    for qi in (17, 67):
        a, b, c, d = imap[qi, :4]
        ci = gg.ClassInfo(*[int(sh.l[s]) for s in (a, b, c, d)])
        cen = [sh.centers[s] for s in (a, b, c, d)]
        ex = [list(sh.exps[sh.prim_off[s]:sh.prim_off[s + 1]]) for s in (a, b, c, d)]
        co = [list(sh.coefs[sh.prim_off[s]:sh.prim_off[s + 1]]) for s in (a, b, c, d)]
        em = emulate(ci, cen, ex, co, True).ravel()
        ref = oracle.eri_block(sh, [a, b, c, d], True).ravel()
        B = oracle.hgp_rounding_bound(sh, [[a, b, c, d]], True)
        assert np.all(np.abs(em - ref) <= np.maximum(1e-13, 4.0 * B))


def test_two_phase_fp64_floor_is_eps_level_when_well_conditioned():
    sh = _pack([[0, 0, 0], [0.5, 0, 0], [0, 0.7, 0], [0, 0, 0.4]], [2, 1, 2, 0], [1, 1, 1, 1],
               [np.array([1.3]), np.array([0.9]), np.array([2.1]), np.array([0.6])], [np.ones(1)] * 4)
    ref = np.abs(oracle.eri_block(sh, [0, 1, 2, 3], True)).max()
    B = oracle.hgp_rounding_bound(sh, [[0, 1, 2, 3]], True)
    assert B.max() < 1e-14 * ref


def test_ablation_variants_generate(tmp_path):
    """Every ablation variant of the generator emits its classes with the routing
    it names: the single-tier variants put every class in one tier, the graph and
    order variants change the emitted lane-tier code, and the product variant
    emits exactly the product sources."""
    from electron_repulsion_integrals_amd.gen import variant
    from electron_repulsion_integrals_amd.gen.emit import generate
    # (pp|pp) and (dd|dd) in the lane-group tiers, (ff|ps) packed on four waves,
    # (fd|fd) in the memory tier; the lane-only variants skip (fd|fd), whose
    # one-quartet-per-lane graph takes minutes to schedule
    cls = [gg.ClassInfo(1, 1, 1, 1), gg.ClassInfo(2, 2, 2, 2), gg.ClassInfo(3, 3, 1, 0), gg.ClassInfo(3, 2, 3, 2)]
    srcs = {}
    for name in variant.VARIANTS:
        prev = variant.set_variant(name)
        try:
            use = cls[:3] if variant.VARIANTS[name].tiers == "lane" else cls
            files, entries = generate(str(tmp_path / name), lmax=4, classes=use)
        finally:
            variant.set_variant(prev)
        tiers = [t for (_, _, _, t, _) in entries]
        if variant.VARIANTS[name].tiers == "memory":
            assert set(tiers) == {"M"}
        elif variant.VARIANTS[name].tiers == "lane":
            assert set(tiers) == {"V"}
            assert all("one quartet per lane" in open(f).read() for f in files[:-1])
        else:
            assert tiers == ["V"] * 6 + ["M"] * 2
        srcs[name] = {os.path.basename(f): open(f).read() for f in files}
    assert srcs["no_dsa"]["eri_c5_s.hip"] != srcs["full"]["eri_c5_s.hip"]
    assert srcs["lane_alg1"]["eri_c5_s.hip"] != srcs["lane_only"]["eri_c5_s.hip"]
    assert srcs["lane_bra_first"]["eri_c5_s.hip"] != srcs["lane_only"]["eri_c5_s.hip"]
    assert srcs["no_sph_fusion"] == srcs["full"]
    from electron_repulsion_integrals_amd.build import GEN_DIR
    for fn, text in srcs["full"].items():
        if fn.startswith("eri_c") and os.path.exists(os.path.join(GEN_DIR, fn)):
            assert open(os.path.join(GEN_DIR, fn)).read() == text, fn
