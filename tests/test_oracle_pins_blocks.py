"""Pins of the oracle's block-wise J/K references and of its Schwarz factors.

oracle.J_blocks and oracle.K_blocks are the references the GPU tests use for J
and K of the 30-atom cluster (Algorithm 2 of "FusionRCG", section III-C: the
integrals are scattered into J and K).  They sum, for the requested blocks,
over every ket pair (J) or every (j, l) shell pair (K) that passes the Schwarz
test, with plain loops.  Here they are checked against two other paths that
share none of that reasoning:
  * with tau = 0, against the plain four-index sums oracle.J_naive /
    oracle.K_naive over every ordered shell quadruple, with no symmetry;
  * with tau > 0, against the unique-quartet digestion (oracle.J_from_quartets /
    K_from_quartets, which use the 8-fold permutation symmetry) over the
    quartets of the screened plan written out by oracle.plan.screened_plan.
oracle.schwarz (S_ij = max |(mu nu|mu nu)| over the (ij|ij) block, the reading
taken for the page's unstated screen) is checked against the closed form of
the Coulomb self-energy of a sum of Gaussian charges for every s-s pair, and
against its definition element by element for every pair.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import plan as oplan
from workloads import make_config


def _density(n, seed):
    rng = np.random.default_rng(seed)
    C = rng.standard_normal((n, max(1, n // 4)))
    return C @ C.T


def _cases():
    return [("C1 Cartesian", make_config(1).shells, False),
            ("3-atom cluster spherical", make_config(3, scale={"natoms": 3}).shells, True)]


@pytest.mark.parametrize("case", [0, 1])
def test_J_blocks_equal_naive_sum(case):
    name, sh, sph = _cases()[case]
    n = sh.nbf(sph)
    D = _density(n, 11 + case)
    Jn = oracle.J_naive(sh, sph, D)
    S = oracle.schwarz(sh, sph)
    bf = oracle.basis_offsets(sh, sph)
    pairs = [(i, j) for i in range(sh.nshell) for j in range(i + 1)]
    blocks = oracle.J_blocks(sh, sph, pairs, D, S, 0.0)
    scale = np.abs(Jn).max()
    for (i, j), blk in zip(pairs, blocks):
        np.testing.assert_allclose(blk, Jn[bf[i]:bf[i + 1], bf[j]:bf[j + 1]], rtol=1e-11, atol=1e-13 * scale,
                                   err_msg=f"{name} pair {(i, j)}")


@pytest.mark.parametrize("case", [0, 1])
def test_K_blocks_equal_naive_sum(case):
    name, sh, sph = _cases()[case]
    n = sh.nbf(sph)
    D = _density(n, 21 + case)
    Kn = oracle.K_naive(sh, sph, D)
    S = oracle.schwarz(sh, sph)
    bf = oracle.basis_offsets(sh, sph)
    pairs = [(i, k) for i in range(sh.nshell) for k in range(sh.nshell)]
    blocks = oracle.K_blocks(sh, sph, pairs, D, S, 0.0)
    scale = np.abs(Kn).max()
    for (i, k), blk in zip(pairs, blocks):
        np.testing.assert_allclose(blk, Kn[bf[i]:bf[i + 1], bf[k]:bf[k + 1]], rtol=1e-11, atol=1e-13 * scale,
                                   err_msg=f"{name} pair {(i, k)}")


def test_screened_J_and_K_blocks_equal_unique_quartet_digestion():
    """tau > 0 on the 3-atom cluster (spherical): a screen that drops about half
    the unique quartets.  J_blocks / K_blocks keep exactly the quartets with
    fl(S_ij S_kl) >= fl(tau^2); the screened plan lists the same quartets in
    canonical form, and the 8-fold digestion of those gives the same J and K."""
    sh = make_config(3, scale={"natoms": 3}).shells
    sph = True
    S = oracle.schwarz(sh, sph)
    tau = float(np.sqrt(np.median(np.outer(S, S))))
    p = oplan.screened_plan(sh.l, sh.nprim, S, tau)
    q = p["index_map"][:, :4]
    ns = sh.nshell
    n_unique = (ns * (ns + 1) // 2) * (ns * (ns + 1) // 2 + 1) // 2
    assert 0.2 * n_unique < len(q) < 0.8 * n_unique, (len(q), n_unique)
    n = sh.nbf(sph)
    D = _density(n, 31)
    flat, off = oracle.eri(sh, q, sph)
    Jq = oracle.J_from_quartets(sh, sph, q, flat, off, D)
    Kq = oracle.K_from_quartets(sh, sph, q, flat, off, D)
    bf = oracle.basis_offsets(sh, sph)
    jp = [(i, j) for i in range(ns) for j in range(i + 1)]
    for (i, j), blk in zip(jp, oracle.J_blocks(sh, sph, jp, D, S, tau)):
        np.testing.assert_allclose(blk, Jq[bf[i]:bf[i + 1], bf[j]:bf[j + 1]], rtol=1e-11,
                                   atol=1e-13 * np.abs(Jq).max(), err_msg=f"J {(i, j)}")
    kp = [(i, k) for i in range(ns) for k in range(ns)]
    for (i, k), blk in zip(kp, oracle.K_blocks(sh, sph, kp, D, S, tau)):
        np.testing.assert_allclose(blk, Kq[bf[i]:bf[i + 1], bf[k]:bf[k + 1]], rtol=1e-11,
                                   atol=1e-13 * np.abs(Kq).max(), err_msg=f"K {(i, k)}")


def _ss_pair_self_energy(sh, i, j):
    """(ij|ij) for two s shells: the product phi_i phi_j is a sum of Gaussian
    charges q_kl exp(-p_kl |r - P_kl|^2) (Gaussian product theorem), with total
    charge Q_kl = c_k c_l exp(-a_k a_l |AB|^2 / p_kl) (pi/p_kl)^(3/2), c the
    normalised coefficients (primitive factor included);
    two such charges interact through Q Q' erf(sqrt(p p'/(p+p')) R) / R, which
    tends to Q Q' 2 sqrt(p p'/(p+p') / pi) at R = 0."""
    ea = sh.exps[sh.prim_off[i]:sh.prim_off[i + 1]]
    eb = sh.exps[sh.prim_off[j]:sh.prim_off[j + 1]]
    ca = oracle.normalize(0, ea, sh.coefs[sh.prim_off[i]:sh.prim_off[i + 1]])
    cb = oracle.normalize(0, eb, sh.coefs[sh.prim_off[j]:sh.prim_off[j + 1]])
    A, B = sh.centers[i], sh.centers[j]
    AB2 = float(np.sum((A - B) ** 2))
    charges = []
    for a, c1 in zip(ea, ca):
        for b, c2 in zip(eb, cb):
            p = a + b
            Q = c1 * c2 * math.exp(-a * b / p * AB2) * (math.pi / p) ** 1.5
            charges.append((Q, p, (a * A + b * B) / p))
    e = 0.0
    for Q1, p1, P1 in charges:
        for Q2, p2, P2 in charges:
            mu = math.sqrt(p1 * p2 / (p1 + p2))
            R = float(np.linalg.norm(P1 - P2))
            e += Q1 * Q2 * (2 * mu / math.sqrt(math.pi) if R < 1e-12 else math.erf(mu * R) / R)
    return e


@pytest.mark.parametrize("case", [0, 1])
def test_schwarz_factors(case):
    name, sh, sph = _cases()[case]
    S = oracle.schwarz(sh, sph)
    ns = sh.nshell
    n_ss = 0
    for i in range(ns):
        for j in range(i + 1):
            p = i * (i + 1) // 2 + j
            blk = oracle.eri_block(sh, [i, j, i, j], sph)
            n = blk.shape[0] * blk.shape[1]
            diag = np.abs(np.diag(blk.reshape(n, n)))
            assert S[p] == diag.max(), (name, i, j)
            if sh.l[i] == 0 and sh.l[j] == 0:
                ref = _ss_pair_self_energy(sh, i, j)
                assert abs(S[p] - ref) <= 1e-12 * ref, (name, i, j, S[p], ref)
                n_ss += 1
    assert n_ss >= 10


def test_J_floor_equals_sum_of_quartet_floors():
    """oracle.hgp_rounding_bound_J (the per-integral two-phase floor propagated
    into J blocks, in matrix form and batched over kets) equals the plain sum
    over the kept ket pairs of f_kl sum_cd B[ab, cd] |D_cd| with B from
    oracle.hgp_rounding_bound quartet by quartet in the library's orientation
    (higher l first, higher index first for equal l), on the 3-atom cluster."""
    sh = make_config(3, scale={"natoms": 3}).shells
    sph = True
    S = oracle.schwarz(sh, sph)
    tau = 1e-6
    n = sh.nbf(sph)
    D = _density(n, 41)
    bf = oracle.basis_offsets(sh, sph)
    ns = sh.nshell
    # three pairs of l >= 1 shells on different atoms with survivors, one pair on
    # one atom, one s-s pair
    far = sorted(((i, j) for i in range(ns) for j in range(i) if sh.l[i] >= 1 and sh.l[j] >= 1
                  and np.any(sh.centers[i] != sh.centers[j])), key=lambda p: -S[p[0] * (p[0] + 1) // 2 + p[1]])
    pairs = far[:3] + [(5, 3), (2, 2)]
    got = oracle.hgp_rounding_bound_J(sh, sph, pairs, D, S, tau)

    def orient(i, j):
        i, j = max(i, j), min(i, j)
        return (j, i) if sh.l[i] < sh.l[j] else (i, j)
    for (i, j), F in zip(pairs, got):
        a, b = orient(i, j)
        pij = max(i, j) * (max(i, j) + 1) // 2 + min(i, j)
        ref = np.zeros((oracle.nfunc(int(sh.l[a]), sph), oracle.nfunc(int(sh.l[b]), sph)))
        for k in range(ns):
            for l in range(k + 1):
                if S[pij] * S[k * (k + 1) // 2 + l] < tau * tau:
                    continue
                c, d = orient(k, l)
                B = oracle.hgp_rounding_bound(sh, [[a, b, c, d]], sph)
                nc, nd = oracle.nfunc(int(sh.l[c]), sph), oracle.nfunc(int(sh.l[d]), sph)
                B = B.reshape(ref.shape[0], ref.shape[1], nc, nd)
                ref += (2.0 if c != d else 1.0) * np.einsum("abcd,cd->ab", B, np.abs(D[bf[c]:bf[c + 1], bf[d]:bf[d + 1]]))
        if a != i:
            ref = ref.T
        np.testing.assert_allclose(F, ref, rtol=1e-12, atol=1e-300)
        assert F.max() > 0
