"""GPU parity of the first-derivative integrals (eri_compute_deriv) against the oracle.

The oracle differentiates each primitive Gaussian in its own four-index
Obara-Saika table (oracle.eri_deriv, pinned by finite differences,
translational invariance and a closed form in test_oracle_pins.py); the
library combines integrals of the neighbouring classes computed by its class
kernels on raised and lowered auxiliary shells.  The two share only the
definition.

Bar, element by element: a derivative element is a difference
P - n M of two integrals of the neighbouring classes (P over the raised shell
with coefficients 2 alpha c, M over the lowered one, n the lowered Cartesian
exponent), each computed to the integral bar of the other tests
(max(1e-10 |x|, 1e-13, 4 B) with B the two-phase fp64 floor of the method),
so |gpu - oracle| <= bar(P) + n bar(M) + 1e-13, with P, M and B taken from the
oracle's own integrals of those auxiliary shells (oracle.eri,
oracle.hgp_rounding_bound).  Where there is no cancellation and no floor this
is the integral bar.
"""
import numpy as np
import pytest

import oracle
from workloads import make_config
from workloads.configs import _pack

from floor_log import FLOOR_FACTOR, record

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def eri():
    import torch
    assert torch.cuda.is_available()
    import electron_repulsion_integrals_amd as E
    E.load()
    return E


def _sub_shells(sh, idx):
    """Shells idx as their own shell set (raw coefficients kept)."""
    cen = [sh.centers[i] for i in idx]
    ls = [int(sh.l[i]) for i in idx]
    ks = [int(sh.nprim[i]) for i in idx]
    ex = [sh.exps[sh.prim_off[i]:sh.prim_off[i + 1]] for i in idx]
    co = [sh.coefs[sh.prim_off[i]:sh.prim_off[i + 1]] for i in idx]
    return _pack(cen, ls, ks, ex, co)


HGP_FLOOR_FACTOR = FLOOR_FACTOR


def _canonical_order(ls):
    """Positions of a quartet in the library's canonical order: a<->b if
    l_a < l_b, c<->d if l_c < l_d, then bra<->ket if pc(bra) < pc(ket)."""
    o = [0, 1, 2, 3]
    if ls[o[0]] < ls[o[1]]:
        o[0], o[1] = o[1], o[0]
    if ls[o[2]] < ls[o[3]]:
        o[2], o[3] = o[3], o[2]

    def pc(a, b):
        return a * (a + 1) // 2 + b
    if pc(ls[o[0]], ls[o[1]]) < pc(ls[o[2]], ls[o[3]]):
        o = [o[2], o[3], o[0], o[1]]
    return o


def deriv_bar(sh, quartets, spherical):
    """Per element: bar(P) + n bar(M) + 1e-13, with bar(x) the integral bar of the
    auxiliary element x (max of 1e-10 |x|, 1e-13 and 4 times the oracle's
    two-phase fp64 floor of that element, as in the integral tests), from the
    oracle's integrals of the raised and lowered auxiliary shells (Cartesian;
    for spherical blocks propagated through |t^(l)|)."""
    q = np.asarray(quartets).reshape(-1, 4)
    out = []
    for row in q:
        sub = _sub_shells(sh, list(row))
        ls = [int(x) for x in sub.l]
        cn = [oracle.normalize(ls[t], sub.exps[sub.prim_off[t]:sub.prim_off[t + 1]],
                               sub.coefs[sub.prim_off[t]:sub.prim_off[t + 1]]) for t in range(4)]
        ex = [sub.exps[sub.prim_off[t]:sub.prim_off[t + 1]] for t in range(4)]
        nc = [oracle.ncart(l) for l in ls]
        mag = np.zeros([4, 3] + nc)
        for p in range(4):
            for sg in (1, -1):
                lp = ls[p] + sg
                if lp < 0:
                    continue
                co = [c.copy() for c in cn]
                co[p] = (2 * ex[p] * cn[p]) if sg > 0 else cn[p]
                ll = list(ls)
                ll[p] = lp
                aux = _pack([sub.centers[t] for t in range(4)], ll, [len(e) for e in ex], ex, co)
                # the integral bar of each auxiliary element: 1e-10 relative, 1e-13
                # absolute, or the two-phase fp64 floor 4 B of the method, B taken
                # for the quartet in the canonical order the library evaluates it in
                order = _canonical_order(ll)
                val = oracle.eri_block(aux, order, False, normalize_=False)
                B = oracle.hgp_rounding_bound(aux, [order], False, normalize_=False).reshape(val.shape)
                blk = np.maximum(np.maximum(1e-10 * np.abs(val), 1e-13), HGP_FLOOR_FACTOR * B)
                blk = np.transpose(blk, np.argsort(order))
                comps = oracle.cart_components(ls[p])
                comps_n = oracle.cart_components(lp)
                for i in range(3):
                    for ci, c in enumerate(comps):
                        t = list(c)
                        t[i] += sg
                        if t[i] < 0:
                            continue
                        j = comps_n.index(tuple(t))
                        src = [slice(None)] * 4
                        src[p] = j
                        dst = [p, i] + [slice(None)] * 4
                        dst[2 + p] = ci
                        w = 1.0 if sg > 0 else c[i]
                        mag[tuple(dst)] += w * blk[tuple(src)]
        if spherical:
            for pos in range(4):
                T = np.abs(np.asarray(oracle.sph_coeffs(ls[pos])))
                mag = np.moveaxis(np.tensordot(T, np.moveaxis(mag, 2 + pos, 0), axes=(1, 0)), 0, 2 + pos)
        out.append(mag.ravel() + 1e-13)
    return np.concatenate(out)


def assert_deriv_parity(got, ref, bar, what):
    err = np.abs(got - ref)
    bad = err > bar
    if bad.any():
        i = int(np.argmax(err / bar))
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} outside the bar; worst at {i}: "
                             f"gpu={got[i]!r} oracle={ref[i]!r} err={err[i]:.3e} bar={bar[i]:.3e}")
    plain = err > np.maximum(1e-10 * np.abs(ref), 1e-13)
    record(what, got.size, int(plain.sum()), 0.0, max_err_over_bar=round(float(np.max(err / bar)) if err.size else 0.0, 4))
    _log(f"  {what}: {got.size} elements, {int(plain.sum())} beyond 1e-10 relative (within the difference bar)")


def run_deriv(E, sh, flags, quartets=None, first=0, count=None):
    import torch
    plan = E.build_quartets(sh, flags, quartets, 0.0)
    imap = plan.index_map().cpu().numpy()
    if count is None:
        count = plan.n_quartets - first
    rows = imap[first:first + count, :4]
    sizes = oracle.block_sizes(sh, rows, bool(flags & 1))
    out = torch.empty(max(12 * int(sizes.sum()), 1), dtype=torch.float64, device="cuda")
    E.compute_deriv(plan, out, first, count)
    torch.cuda.synchronize()
    return plan, out[:12 * int(sizes.sum())].cpu().numpy(), rows


def _mixed(seed, nshell, nq, lmax, kmax):
    rng = np.random.default_rng(seed)
    cen = rng.uniform(0, 5, (nshell, 3))
    ls = rng.integers(0, lmax + 1, nshell)
    ks = rng.integers(1, kmax + 1, nshell)
    ex = [np.exp(rng.uniform(np.log(0.15), np.log(20.0), k)) for k in ks]
    co = [rng.uniform(0.1, 1.0, k) for k in ks]
    sh = _pack(cen, ls, ks, ex, co)
    q = rng.integers(0, nshell, (nq, 4)).astype(np.int32)
    return sh, q


def _mixed_g(seed, nshell, nq, kmax, cap=8e6):
    """Random shells up to l = 4 (a quarter of them g) and nq quartets that each
    hold at least one g shell, limited to quartets whose oracle derivative table
    (every index one higher) stays below ``cap`` doubles."""
    def tri(l):
        return (l + 1) * (l + 2) * (l + 3) // 6
    rng = np.random.default_rng(seed)
    cen = rng.uniform(0, 5, (nshell, 3))
    ls = rng.integers(0, 5, nshell)
    ls[: nshell // 4] = 4
    ks = rng.integers(1, kmax + 1, nshell)
    ex = [np.exp(rng.uniform(np.log(0.15), np.log(20.0), k)) for k in ks]
    co = [rng.uniform(0.1, 1.0, k) for k in ks]
    sh = _pack(cen, ls, ks, ex, co)
    out = []
    while len(out) < nq:
        q = rng.integers(0, nshell, 4)
        l4 = ls[q]
        if 4 not in l4 or np.prod([tri(int(l) + 1) for l in l4]) * (int(l4.sum()) + 5) > cap:
            continue
        out.append(q)
    return sh, np.array(out, dtype=np.int32)


def test_deriv_tiny_molecule_cartesian(eri):
    """All 666 unique quartets of the s/p tiny molecule, every derivative block."""
    _log("case: derivatives, tiny molecule, Cartesian")
    w = make_config(1)
    plan, got, rows = run_deriv(eri, w.shells, 0)
    ref, _ = oracle.eri_deriv(w.shells, rows, False)
    assert_deriv_parity(got, ref, deriv_bar(w.shells, rows, False), "tiny molecule derivatives")


@pytest.mark.parametrize("spherical", [False, True])
def test_deriv_mixed_classes_l3(eri, spherical):
    """Random explicit batch over classes up to l = 3 (K <= 2): ragged class
    blocks, every canonical permutation the plan applies."""
    _log(f"case: derivatives, mixed l<=3 batch, spherical={spherical}")
    sh, q = _mixed(31, 24, 300, 3, 2)
    plan, got, rows = run_deriv(eri, sh, 1 if spherical else 0, q)
    ref, _ = oracle.eri_deriv(sh, rows, spherical)
    assert_deriv_parity(got, ref, deriv_bar(sh, rows, spherical), f"mixed l<=3 derivatives sph={spherical}")


@pytest.mark.parametrize("spherical", [False, True])
def test_deriv_g_shells(eri, spherical):
    """Quartets with g shells (K <= 2): the raised shell reaches l = 5, which the
    library's raised-shell classes (Cartesian kernels) compute; against the
    oracle's derivatives (its four-index table one higher on every index)."""
    _log(f"case: derivatives with g shells, spherical={spherical}")
    sh, q = _mixed_g(43, 16, 60, 2)
    plan, got, rows = run_deriv(eri, sh, 1 if spherical else 0, q)
    assert max(int(sh.l[s]) for s in rows.ravel()) == 4
    ref, _ = oracle.eri_deriv(sh, rows, spherical)
    assert_deriv_parity(got, ref, deriv_bar(sh, rows, spherical), f"g-shell derivatives sph={spherical}")


def test_deriv_slot_range_and_translational_invariance(eri):
    """A slot range equals the same slots of the whole plan; the four centre
    derivatives of every block sum to zero within the sum of their bars."""
    _log("case: derivatives, slot range and invariance")
    sh, q = _mixed(37, 16, 120, 2, 3)
    plan, whole, rows = run_deriv(eri, sh, 1, q)
    sizes = 12 * oracle.block_sizes(sh, rows, True)
    off = np.concatenate([[0], np.cumsum(sizes)])
    _, part, rows2 = run_deriv(eri, sh, 1, q, first=17, count=41)
    np.testing.assert_array_equal(rows2, rows[17:58])
    np.testing.assert_array_equal(part, whole[off[17]:off[58]])
    bar = deriv_bar(sh, rows, True)
    for t in range(len(rows)):
        blk = whole[off[t]:off[t + 1]].reshape(4, 3, -1)
        lim = bar[off[t]:off[t + 1]].reshape(4, 3, -1).sum(axis=0)
        assert np.all(np.abs(blk.sum(axis=0)) <= lim), t


def test_deriv_cluster_subset(eri):
    """Screened 4-atom SVP-like cluster (spherical), a seeded sample of slots
    of the plan, compared with the oracle."""
    _log("case: derivatives, 4-atom cluster sample")
    w = make_config(3, scale={"natoms": 4})
    import torch
    plan = eri.build_quartets(w.shells, 1, None, w.tau)
    rng = np.random.default_rng(5)
    first = int(rng.integers(0, plan.n_quartets - 200))
    imap = plan.index_map().cpu().numpy()
    rows = imap[first:first + 200, :4]
    sizes = oracle.block_sizes(w.shells, rows, True)
    out = torch.empty(12 * int(sizes.sum()), dtype=torch.float64, device="cuda")
    eri.compute_deriv(plan, out, first, 200)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref, _ = oracle.eri_deriv(w.shells, rows, True)
    assert_deriv_parity(got, ref, deriv_bar(w.shells, rows, True), "cluster derivative sample")


def test_deriv_errors(eri):
    """Short output buffers and more than 2^24 slots are rejected; nothing is
    written then."""
    import torch
    from electron_repulsion_integrals_amd import EriError
    sh, q = _mixed(41, 6, 10, 1, 1)
    plan = eri.build_quartets(sh, 0, q, 0.0)
    small = torch.zeros(3, dtype=torch.float64, device="cuda")
    with pytest.raises(EriError) as e:
        eri.compute_deriv(plan, small)
    assert e.value.code == -3
    assert float(small.abs().sum()) == 0.0
    with pytest.raises(EriError) as e:
        eri.compute_deriv(plan, small, 0, (1 << 24) + 1)
    assert e.value.code == -1
