"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a closed form, an identity of
the mathematics, a library routine (mpmath, scipy), or a structural count from
"FusionRCG: Orchestrating Recursive Computation Graphs across GPU Memory
Hierarchies" (cited by section).  Together they are chosen so that a dropped
term, a wrong sign or index, or a transposed operand in the oracle fails one
of them (tests/test_oracle_mutants.py plants such mistakes and checks that).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import plan as oplan
from workloads import make_config
from workloads.configs import _pack

mpmath = pytest.importorskip("mpmath")


def shells_from(spec, normalize_coefs=None):
    """spec: list of (centre[3], l, [alphas], [coefs])."""
    centers = [s[0] for s in spec]
    ls = [s[1] for s in spec]
    ks = [len(s[2]) for s in spec]
    ex = [np.asarray(s[2], dtype=float) for s in spec]
    co = [np.asarray(s[3] if len(s) > 3 else [1.0] * len(s[2]), dtype=float) for s in spec]
    return _pack(centers, ls, ks, ex, co)


# --------------------------------------------------------------------------
# Boys function
# --------------------------------------------------------------------------

def test_boys_at_zero():
    F = oracle.boys(24, 0.0)
    for m in range(25):
        assert F[m] == pytest.approx(1.0 / (2 * m + 1), rel=1e-15)


@pytest.mark.parametrize("T", [1e-12, 1e-6, 0.3, 1.0, 7.5, 20.0, 36.0, 49.99, 50.01, 80.0, 1e3, 1e5, 4e7])
def test_boys_f0_is_erf(T):
    F = oracle.boys(0, T)
    ref = 0.5 * math.sqrt(math.pi / T) * math.erf(math.sqrt(T))
    assert F[0] == pytest.approx(ref, rel=2e-15)


@pytest.mark.parametrize("T", [1e-10, 1e-3, 0.1, 1.0, 4.9, 12.0, 30.0, 49.999, 50.001, 60.0, 300.0, 1e4, 4e7])
def test_boys_vs_mpmath(T):
    """F_m(T) = gamma_lower(m+1/2, T) / (2 T^(m+1/2)), evaluated by mpmath at 40 digits."""
    mpmath.mp.dps = 40
    F = oracle.boys(20, T)
    for m in range(21):
        ref = float(mpmath.gammainc(m + mpmath.mpf(1) / 2, 0, T) / (2 * mpmath.mpf(T) ** (m + mpmath.mpf(1) / 2)))
        assert F[m] == pytest.approx(ref, rel=2e-14), (m, T)


def test_boys_recursion_identity():
    """(2m+1) F_m = 2T F_{m+1} + exp(-T) at every order, both branches."""
    for T in [0.01, 2.0, 45.0, 55.0, 500.0]:
        F = oracle.boys(16, T)
        for m in range(16):
            lhs = (2 * m + 1) * F[m]
            rhs = 2 * T * F[m + 1] + math.exp(-T)
            assert lhs == pytest.approx(rhs, rel=1e-13)


# --------------------------------------------------------------------------
# (ss|ss) closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("alpha", [0.1, 1.0, 3.7, 250.0])
def test_ssss_one_centre(alpha):
    """Four normalised s Gaussians on one centre, one exponent: 2 sqrt(alpha/pi)."""
    sh = shells_from([([0.3, -0.2, 1.1], 0, [alpha])] * 4)
    v = oracle.eri_block(sh, [0, 1, 2, 3], False)[0, 0, 0, 0]
    assert v == pytest.approx(2.0 * math.sqrt(alpha / math.pi), rel=1e-14)


@pytest.mark.parametrize("aA,aB,R", [(1.0, 1.0, 0.5), (0.3, 7.0, 2.0), (5.0, 0.05, 11.0), (40.0, 60.0, 1e-3)])
def test_ssss_two_centre_charge_distributions(aA, aB, R):
    """(s_A s_A|s_B s_B) is the Coulomb energy of two unit Gaussian charges of
    exponents 2aA and 2aB a distance R apart: erf(sqrt(p q/(p+q)) R) / R."""
    sh = shells_from([([0, 0, 0], 0, [aA]), ([0, 0, 0], 0, [aA]), ([0, 0, R], 0, [aB]), ([0, 0, R], 0, [aB])])
    v = oracle.eri_block(sh, [0, 1, 2, 3], False)[0, 0, 0, 0]
    p, q = 2 * aA, 2 * aB
    ref = math.erf(math.sqrt(p * q / (p + q)) * R) / R
    assert v == pytest.approx(ref, rel=1e-13)


def test_ssss_four_centre_gaussian_charges():
    """Contracted (ss|ss) over four centres via the Gaussian product theorem:
    each product s_A s_B is a Gaussian charge of exponent alpha+beta, weight
    exp(-alpha beta AB^2/(alpha+beta)) (pi/(alpha+beta))^1.5 at P; two such
    charges interact through erf(sqrt(p q/(p+q)) R_PQ)/R_PQ."""
    rng = np.random.default_rng(7)
    spec = []
    for t in range(4):
        k = 2 + t % 2
        spec.append((rng.uniform(-2, 2, 3), 0, list(np.exp(rng.uniform(-1, 2, k))), list(rng.uniform(0.2, 1, k))))
    sh = shells_from(spec)
    v = oracle.eri_block(sh, [0, 1, 2, 3], False, normalize_=False)[0, 0, 0, 0]
    ref = 0.0
    for (A, _, al1, c1), (B, _, al2, c2), (C, _, al3, c3), (D, _, al4, c4) in [spec]:
        for a, ca in zip(al1, c1):
            for b, cb in zip(al2, c2):
                p = a + b
                P = (a * np.asarray(A) + b * np.asarray(B)) / p
                wp = math.exp(-a * b / p * np.sum((np.asarray(A) - B) ** 2)) * (math.pi / p) ** 1.5
                for c, ccc in zip(al3, c3):
                    for d, cd in zip(al4, c4):
                        q = c + d
                        Q = (c * np.asarray(C) + d * np.asarray(D)) / q
                        wq = math.exp(-c * d / q * np.sum((np.asarray(C) - D) ** 2)) * (math.pi / q) ** 1.5
                        R = float(np.linalg.norm(P - Q))
                        ref += ca * cb * ccc * cd * wp * wq * math.erf(math.sqrt(p * q / (p + q)) * R) / R
    assert v == pytest.approx(ref, rel=1e-13)


# --------------------------------------------------------------------------
# Finite differences with respect to the centres (raw primitives)
# --------------------------------------------------------------------------

def _fd_case(ls, pos, axis, seed):
    """d/dX_axis of (ab|cd) for the centre of index `pos` equals
    2 alpha (.. x+1 ..) - x_axis (.. x-1 ..) for raw primitives x^a exp(-alpha r^2)."""
    rng = np.random.default_rng(seed)
    cents = [rng.uniform(-1.5, 1.5, 3) for _ in range(4)]
    alphas = [float(np.exp(rng.uniform(np.log(0.3), np.log(3.0)))) for _ in range(4)]

    def block(lvec, cvec):
        sh = shells_from([(cvec[t], lvec[t], [alphas[t]]) for t in range(4)])
        return oracle.eri_block(sh, [0, 1, 2, 3], False, normalize_=False)

    h = 2e-3

    def deriv():
        out = []
        for hh in (h, h / 2):
            cp = [c.copy() for c in cents]
            cm = [c.copy() for c in cents]
            cp[pos][axis] += hh
            cm[pos][axis] -= hh
            out.append((block(ls, cp) - block(ls, cm)) / (2 * hh))
        return (4 * out[1] - out[0]) / 3  # Richardson extrapolation

    num = deriv()
    up = list(ls)
    up[pos] += 1
    Bup = block(up, cents)
    Bdn = None
    if ls[pos] > 0:
        dn = list(ls)
        dn[pos] -= 1
        Bdn = block(dn, cents)
    comps = oracle.cart_components(ls[pos])
    comps_up = oracle.cart_components(ls[pos] + 1)
    comps_dn = oracle.cart_components(ls[pos] - 1) if ls[pos] > 0 else []
    ana = np.zeros_like(num)
    for ci, c in enumerate(comps):
        cu = list(c)
        cu[axis] += 1
        iu = comps_up.index(tuple(cu))
        sl = [slice(None)] * 4
        sl[pos] = ci
        slu = [slice(None)] * 4
        slu[pos] = iu
        val = 2 * alphas[pos] * Bup[tuple(slu)]
        if c[axis] > 0:
            cd = list(c)
            cd[axis] -= 1
            idn = comps_dn.index(tuple(cd))
            sld = [slice(None)] * 4
            sld[pos] = idn
            val = val - c[axis] * Bdn[tuple(sld)]
        ana[tuple(sl)] = val
    scale = max(1.0, float(np.abs(ana).max()))
    np.testing.assert_allclose(num, ana, rtol=0, atol=2e-8 * scale)


@pytest.mark.parametrize("ls", [(0, 0, 0, 0), (1, 0, 0, 0), (0, 1, 0, 0), (1, 1, 1, 1), (2, 1, 0, 1), (2, 2, 1, 1),
                                (0, 0, 2, 2), (3, 1, 2, 0), (3, 3, 2, 2), (4, 0, 0, 0), (4, 2, 1, 3)])
@pytest.mark.parametrize("pos", [0, 1, 2, 3])
def test_finite_difference_centres(ls, pos):
    for axis in range(3):
        _fd_case(ls, pos, axis, seed=100 * pos + 10 * axis + sum(ls))


# --------------------------------------------------------------------------
# First derivatives with respect to the centres (oracle.eri_deriv)
# --------------------------------------------------------------------------

def _shifted(sh, pos, axis, h):
    c = np.array(sh.centers, dtype=float).copy()
    c[pos, axis] += h
    return shells_from([(c[t], int(sh.l[t]), list(sh.exps[sh.prim_off[t]:sh.prim_off[t + 1]]),
                         list(sh.coefs[sh.prim_off[t]:sh.prim_off[t + 1]])) for t in range(4)])


@pytest.mark.parametrize("ls,spherical", [((0, 0, 0, 0), False), ((1, 0, 0, 0), False), ((1, 1, 1, 0), False),
                                          ((2, 1, 0, 1), True), ((2, 2, 1, 1), False), ((3, 1, 2, 0), True),
                                          ((3, 3, 2, 2), False), ((4, 1, 2, 0), True), ((4, 4, 1, 0), False)])
def test_derivative_finite_differences(ls, spherical):
    """Each of the 12 derivative blocks against a fourth-order central
    difference of the integrals, moving one centre along one axis (contracted,
    normalised shells on four distinct centres)."""
    sh = _random_shells(ls, seed=41 + sum(ls) + 7 * spherical)
    d = oracle.eri_deriv_block(sh, [0, 1, 2, 3], spherical)
    h = 1e-3
    scale = max(1e-3, float(np.abs(d).max()))
    for pos in range(4):
        for axis in range(3):
            f = [oracle.eri_block(_shifted(sh, pos, axis, s * h), [0, 1, 2, 3], spherical) for s in (2, 1, -1, -2)]
            num = (-f[0] + 8 * f[1] - 8 * f[2] + f[3]) / (12 * h)
            np.testing.assert_allclose(d[pos, axis], num, rtol=0, atol=1e-8 * scale)


@pytest.mark.parametrize("ls", [(1, 0, 0, 0), (2, 1, 1, 0), (3, 2, 2, 1), (2, 2, 2, 2)])
def test_derivative_translational_invariance(ls):
    """Moving all four centres together leaves every integral unchanged, so the
    four centre derivatives along each axis sum to zero."""
    sh = _random_shells(ls, seed=13 + sum(ls))
    d = oracle.eri_deriv_block(sh, [0, 1, 2, 3], False)
    total = d.sum(axis=0)
    assert np.abs(total).max() <= 1e-12 * np.abs(d).max()


@pytest.mark.parametrize("aA,aB,R", [(1.0, 1.0, 0.5), (0.3, 7.0, 2.0), (5.0, 0.05, 6.0)])
def test_derivative_two_centre_closed_form(aA, aB, R):
    """(s_A s_A|s_B s_B) = erf(sqrt(rho) R)/R with rho = p q/(p+q), p = 2 aA,
    q = 2 aB (the two-centre pin above); B lies at +R along z, so the A
    derivatives along z sum to -d/dR and the B derivatives to +d/dR of it, and
    the x, y derivatives vanish."""
    sh = shells_from([([0, 0, 0], 0, [aA]), ([0, 0, 0], 0, [aA]), ([0, 0, R], 0, [aB]), ([0, 0, R], 0, [aB])])
    d = oracle.eri_deriv_block(sh, [0, 1, 2, 3], False)[..., 0, 0, 0, 0]
    p, q = 2 * aA, 2 * aB
    rho = p * q / (p + q)
    dfdR = 2 * math.sqrt(rho / math.pi) * math.exp(-rho * R * R) / R - math.erf(math.sqrt(rho) * R) / R ** 2
    assert d[0, 2] + d[1, 2] == pytest.approx(-dfdR, rel=1e-12)
    assert d[2, 2] + d[3, 2] == pytest.approx(dfdR, rel=1e-12)
    assert np.abs(d[:, :2]).max() <= 1e-15


# --------------------------------------------------------------------------
# Symmetries and invariances
# --------------------------------------------------------------------------

def _random_shells(ls, seed, K=2, spherical_range=(0.2, 4.0)):
    rng = np.random.default_rng(seed)
    spec = []
    for t, l in enumerate(ls):
        spec.append((rng.uniform(-2, 2, 3), l, list(np.exp(rng.uniform(np.log(spherical_range[0]), np.log(spherical_range[1]), K))),
                     list(rng.uniform(0.1, 1.0, K))))
    return shells_from(spec)


PERMS = [((0, 1, 2, 3), (0, 1, 2, 3)), ((1, 0, 2, 3), (1, 0, 2, 3)), ((0, 1, 3, 2), (0, 1, 3, 2)),
         ((1, 0, 3, 2), (1, 0, 3, 2)), ((2, 3, 0, 1), (2, 3, 0, 1)), ((3, 2, 0, 1), (2, 3, 1, 0)),
         ((2, 3, 1, 0), (3, 2, 0, 1)), ((3, 2, 1, 0), (3, 2, 1, 0))]


@pytest.mark.parametrize("ls", [(1, 0, 0, 0), (1, 1, 1, 0), (2, 1, 1, 0), (2, 2, 1, 1), (3, 2, 1, 0), (2, 2, 2, 2), (4, 1, 2, 0)])
@pytest.mark.parametrize("spherical", [False, True])
def test_eightfold_symmetry(ls, spherical):
    """(ab|cd) = (ba|cd) = (ab|dc) = (ba|dc) = (cd|ab) = (dc|ab) = (cd|ba) = (dc|ba),
    each permutation evaluated separately (the recurrence is not symmetric in
    construction: it always lowers the first non-zero index)."""
    sh = _random_shells(ls, seed=sum(ls) * 7 + 1)
    ref = oracle.eri_block(sh, [0, 1, 2, 3], spherical)
    for order, axes in PERMS:
        blk = oracle.eri_block(sh, list(order), spherical)
        # blk[i,j,k,l] is indexed by the shells in `order`; bring back to (0,1,2,3)
        back = np.transpose(blk, np.argsort(order))
        np.testing.assert_allclose(back, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())


@pytest.mark.parametrize("ls", [(1, 1, 0, 0), (2, 1, 2, 0), (3, 3, 1, 1), (2, 2, 2, 2)])
def test_translation_invariance(ls):
    sh = _random_shells(ls, seed=11 + sum(ls))
    ref = oracle.eri_block(sh, [0, 1, 2, 3], False)
    sh2 = shells_from([(sh.centers[t] + np.array([3.7, -1.25, 5.5]), int(sh.l[t]),
                        list(sh.exps[sh.prim_off[t]:sh.prim_off[t + 1]]),
                        list(sh.coefs[sh.prim_off[t]:sh.prim_off[t + 1]])) for t in range(4)])
    got = oracle.eri_block(sh2, [0, 1, 2, 3], False)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def _rotation(seed):
    rng = np.random.default_rng(seed)
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


@pytest.mark.parametrize("ls", [(1, 0, 0, 0), (1, 1, 1, 1), (2, 0, 1, 0), (2, 2, 2, 2), (3, 2, 1, 1), (4, 3, 0, 2)])
def test_rotation_invariance_spherical_norm(ls):
    """Real solid harmonics of one l span a rotation-invariant space and are
    orthonormal, so the Frobenius norm of a spherical block is unchanged when
    all centres rotate.  (Cartesian d or higher components are not orthonormal,
    so their block norm is not invariant -- this pins the transform.)"""
    sh = _random_shells(ls, seed=3 + sum(ls))
    R = _rotation(sum(ls) + 5)
    sh2 = shells_from([(R @ sh.centers[t], int(sh.l[t]), list(sh.exps[sh.prim_off[t]:sh.prim_off[t + 1]]),
                        list(sh.coefs[sh.prim_off[t]:sh.prim_off[t + 1]])) for t in range(4)])
    a = oracle.eri_block(sh, [0, 1, 2, 3], True)
    b = oracle.eri_block(sh2, [0, 1, 2, 3], True)
    assert np.linalg.norm(b) == pytest.approx(np.linalg.norm(a), rel=1e-11)


def test_rotation_p_shell_is_a_vector():
    """A p shell rotates as a vector: (p s|s s)(R r) = R (p s|s s)(r)."""
    sh = _random_shells((1, 0, 0, 0), seed=5)
    R = _rotation(9)
    sh2 = shells_from([(R @ sh.centers[t], int(sh.l[t]), list(sh.exps[sh.prim_off[t]:sh.prim_off[t + 1]]),
                        list(sh.coefs[sh.prim_off[t]:sh.prim_off[t + 1]])) for t in range(4)])
    a = oracle.eri_block(sh, [0, 1, 2, 3], False)[:, 0, 0, 0]
    b = oracle.eri_block(sh2, [0, 1, 2, 3], False)[:, 0, 0, 0]
    np.testing.assert_allclose(b, R @ a, rtol=1e-11, atol=1e-13)


def test_schwarz_inequality_c1():
    w = make_config(1)
    sh = w.shells
    ns = sh.nshell
    q = [(i, j, k, l) for i in range(ns) for j in range(ns) for k in range(ns) for l in range(ns)]
    flat, off = oracle.eri(sh, q, False)
    n = [oracle.ncart(int(x)) for x in sh.l]
    blocks = {}
    for t, (i, j, k, l) in enumerate(q):
        blocks[(i, j, k, l)] = flat[off[t]: off[t] + n[i] * n[j] * n[k] * n[l]].reshape(n[i], n[j], n[k], n[l])
    for (i, j, k, l), B in blocks.items():
        dij = np.einsum("abab->ab", blocks[(i, j, i, j)])
        dkl = np.einsum("cdcd->cd", blocks[(k, l, k, l)])
        bound = np.sqrt(np.abs(dij)[:, :, None, None] * np.abs(dkl)[None, None, :, :])
        assert np.all(np.abs(B) <= bound * (1 + 1e-12) + 1e-15)


def _full_eri_matrix(sh, spherical):
    ns = sh.nshell
    bf = oracle.basis_offsets(sh, spherical)
    N = int(bf[-1])
    q = [(i, j, k, l) for i in range(ns) for j in range(ns) for k in range(ns) for l in range(ns)]
    flat, off = oracle.eri(sh, q, spherical)
    M = np.zeros((N, N, N, N))
    for t, (i, j, k, l) in enumerate(q):
        n = [bf[x + 1] - bf[x] for x in (i, j, k, l)]
        M[bf[i]:bf[i + 1], bf[j]:bf[j + 1], bf[k]:bf[k + 1], bf[l]:bf[l + 1]] = \
            flat[off[t]: off[t] + np.prod(n)].reshape(n)
    return M


def test_eri_matrix_positive_semidefinite_c1():
    """(mu nu|la si) as a matrix over pairs is a Coulomb Gram matrix: PSD."""
    sh = make_config(1).shells
    M = _full_eri_matrix(sh, False)
    N = M.shape[0]
    ev = np.linalg.eigvalsh(M.reshape(N * N, N * N))
    assert ev.min() >= -1e-12 * ev.max()


# --------------------------------------------------------------------------
# Normalisation and spherical transform
# --------------------------------------------------------------------------

@pytest.mark.parametrize("l", [0, 1, 2, 3, 4])
def test_normalised_shell_has_unit_norm_by_quadrature(l):
    """Self-overlap of the contracted x^l component, by 1-D numerical quadrature."""
    from scipy.integrate import quad
    rng = np.random.default_rng(l)
    K = 4
    al = np.exp(rng.uniform(np.log(0.1), np.log(50), K))
    c = rng.uniform(0.1, 1.0, K)
    cn = oracle.normalize(l, al, c)
    tot = 0.0
    for a, ca in zip(al, cn):
        for b, cb in zip(al, cn):
            p = a + b
            ix = quad(lambda x: x ** (2 * l) * math.exp(-p * x * x), -np.inf, np.inf, epsabs=0, epsrel=1e-13)[0]
            iy = quad(lambda x: math.exp(-p * x * x), -np.inf, np.inf, epsabs=0, epsrel=1e-13)[0]
            tot += ca * cb * ix * iy * iy
    assert tot == pytest.approx(1.0, rel=1e-10)


@pytest.mark.parametrize("l", [0, 1, 2, 3, 4])
def test_primitive_weights_by_quadrature(l):
    """Raw coefficients multiply individually normalised primitives: the ratio of
    two normalised coefficients is c1 N(a1) / (c2 N(a2)) with
    N(a) = (int x^(2l) exp(-2 a r^2) d^3r)^(-1/2) computed by quadrature."""
    from scipy.integrate import quad
    al = np.array([0.37, 6.1])
    c = np.array([0.8, 0.45])
    cn = oracle.normalize(l, al, c)

    def N(a):
        ix = quad(lambda x: x ** (2 * l) * math.exp(-2 * a * x * x), -np.inf, np.inf, epsabs=0, epsrel=1e-13)[0]
        iy = quad(lambda x: math.exp(-2 * a * x * x), -np.inf, np.inf, epsabs=0, epsrel=1e-13)[0]
        return 1.0 / math.sqrt(ix * iy * iy)

    assert cn[0] / cn[1] == pytest.approx(c[0] * N(al[0]) / (c[1] * N(al[1])), rel=1e-10)


def _cart_overlap_matrix(l):
    comps = oracle.cart_components(l)

    def g(n):  # int x^n exp(-x^2) dx up to a common factor: (n-1)!! / 2^(n/2)
        if n % 2:
            return 0.0
        r = 1.0
        for k in range(n - 1, 0, -2):
            r *= k
        return r / 2 ** (n / 2)

    S = np.array([[g(p[0] + q[0]) * g(p[1] + q[1]) * g(p[2] + q[2]) for q in comps] for p in comps])
    return S / g(2 * l)


@pytest.mark.parametrize("l", [0, 1, 2, 3, 4, 5, 6])
def test_spherical_rows_orthonormal(l):
    T = oracle.sph_coeffs(l)
    S = _cart_overlap_matrix(l)
    np.testing.assert_allclose(T @ S @ T.T, np.eye(2 * l + 1), atol=1e-13)


@pytest.mark.parametrize("l", [1, 2, 3, 4, 5])
def test_spherical_rows_are_harmonic(l):
    """Each row, read as a polynomial in x, y, z, has zero Laplacian."""
    T = oracle.sph_coeffs(l)
    comps = oracle.cart_components(l)
    lower = oracle.cart_components(l - 2) if l >= 2 else []
    for row in T:
        lap = {c: 0.0 for c in lower}
        for coef, (i, j, k) in zip(row, comps):
            for ax, e in enumerate((i, j, k)):
                if e >= 2:
                    n = [i, j, k]
                    n[ax] -= 2
                    lap[tuple(n)] += coef * e * (e - 1)
        assert all(abs(v) < 1e-12 for v in lap.values())


def test_spherical_d_shell_known_form():
    """d, m = 0 is proportional to 2z^2 - x^2 - y^2, m = 2 to x^2 - y^2; sign
    convention: the z^l / x^|m| monomial is positive."""
    T = oracle.sph_coeffs(2)  # columns xx xy xz yy yz zz
    r0 = T[2]
    assert r0[5] > 0 and r0[0] == pytest.approx(-0.5 * r0[5]) and r0[3] == pytest.approx(-0.5 * r0[5])
    r2 = T[4]
    assert r2[0] > 0 and r2[3] == pytest.approx(-r2[0]) and abs(r2[5]) < 1e-15
    assert T[0][1] > 0 and T[1][4] > 0 and T[3][2] > 0  # xy, yz, xz


# --------------------------------------------------------------------------
# J and structural counts
# --------------------------------------------------------------------------

def test_J_unique_quartets_equals_naive_sum_c1():
    w = make_config(1)
    sh = w.shells
    N = sh.nbf(False)
    rng = np.random.default_rng(3)
    C = rng.standard_normal((N, N // 4))
    D = C @ C.T
    Jn = oracle.J_naive(sh, False, D)
    ns = sh.nshell
    q = [(i, j, k, l) for i in range(ns) for j in range(i + 1) for k in range(ns) for l in range(k + 1)
         if i * (i + 1) // 2 + j >= k * (k + 1) // 2 + l]
    flat, off = oracle.eri(sh, q, False)
    Ju = oracle.J_from_quartets(sh, False, q, flat, off, D)
    np.testing.assert_allclose(Ju, Jn, rtol=1e-12, atol=1e-12 * np.abs(Jn).max())
    np.testing.assert_allclose(Jn, Jn.T, rtol=1e-12, atol=1e-13 * np.abs(Jn).max())
    assert np.trace(D @ Jn) >= 0


def test_J_spherical_equals_transformed_cartesian():
    """J in the spherical basis = T J_cart(D_cart = T^T D T) T^T for the block-diagonal T."""
    w = make_config(1)
    sh = w.shells
    Ns, Nc = sh.nbf(True), sh.nbf(False)
    Tb = np.zeros((Ns, Nc))
    bs, bc = oracle.basis_offsets(sh, True), oracle.basis_offsets(sh, False)
    for s in range(sh.nshell):
        Tb[bs[s]:bs[s + 1], bc[s]:bc[s + 1]] = oracle.sph_coeffs(int(sh.l[s]))
    rng = np.random.default_rng(4)
    C = rng.standard_normal((Ns, 3))
    D = C @ C.T
    Js = oracle.J_naive(sh, True, D)
    Jc = oracle.J_naive(sh, False, Tb.T @ D @ Tb)
    np.testing.assert_allclose(Js, Tb @ Jc @ Tb.T, rtol=1e-11, atol=1e-12 * np.abs(Js).max())


def _c1_unique_quartets(sh):
    ns = sh.nshell
    return [(i, j, k, l) for i in range(ns) for j in range(i + 1) for k in range(ns) for l in range(k + 1)
            if i * (i + 1) // 2 + j >= k * (k + 1) // 2 + l]


def test_K_unique_quartets_equals_naive_sum_c1():
    """Exchange K_mu,nu = sum (mu la|nu si) D_la,si: the unique-quartet form (every
    distinct permutation of a quartet once) against the plain four-index sum."""
    w = make_config(1)
    sh = w.shells
    N = sh.nbf(False)
    rng = np.random.default_rng(5)
    C = rng.standard_normal((N, N // 4))
    D = C @ C.T
    Kn = oracle.K_naive(sh, False, D)
    q = _c1_unique_quartets(sh)
    flat, off = oracle.eri(sh, q, False)
    Ku = oracle.K_from_quartets(sh, False, q, flat, off, D)
    np.testing.assert_allclose(Ku, Kn, rtol=1e-12, atol=1e-12 * np.abs(Kn).max())
    np.testing.assert_allclose(Kn, Kn.T, rtol=1e-12, atol=1e-13 * np.abs(Kn).max())


def test_K_against_J_energies():
    """One orbital, D = c c^T: c^T K c = c^T J c (both are (cc|cc)).  Several
    orbitals: 0 <= tr(D K) <= tr(D J) (the antisymmetrised pair density is
    non-negative)."""
    w = make_config(1)
    sh = w.shells
    N = sh.nbf(False)
    rng = np.random.default_rng(6)
    c = rng.standard_normal(N)
    D1 = np.outer(c, c)
    J1, K1 = oracle.J_naive(sh, False, D1), oracle.K_naive(sh, False, D1)
    assert c @ K1 @ c == pytest.approx(c @ J1 @ c, rel=1e-12)
    C = rng.standard_normal((N, 5))
    D = C @ C.T
    eJ, eK = np.trace(D @ oracle.J_naive(sh, False, D)), np.trace(D @ oracle.K_naive(sh, False, D))
    assert 0.0 < eK < eJ


def test_K_spherical_equals_transformed_cartesian():
    w = make_config(1)
    sh = w.shells
    Ns, Nc = sh.nbf(True), sh.nbf(False)
    Tb = np.zeros((Ns, Nc))
    bs, bc = oracle.basis_offsets(sh, True), oracle.basis_offsets(sh, False)
    for s in range(sh.nshell):
        Tb[bs[s]:bs[s + 1], bc[s]:bc[s + 1]] = oracle.sph_coeffs(int(sh.l[s]))
    rng = np.random.default_rng(7)
    C = rng.standard_normal((Ns, 3))
    D = C @ C.T
    Ks = oracle.K_naive(sh, True, D)
    Kc = oracle.K_naive(sh, False, Tb.T @ D @ Tb)
    np.testing.assert_allclose(Ks, Tb @ Kc @ Tb.T, rtol=1e-11, atol=1e-12 * np.abs(Ks).max())


def _golden(name):
    import os
    vals = {}
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_structural_counts_from_the_page():
    g = _golden("structure.txt")
    classes = {oplan.class_id(max(oplan.pair_class(a, b), oplan.pair_class(c, d)),
                              min(oplan.pair_class(a, b), oplan.pair_class(c, d)))
               for a in range(5) for b in range(5) for c in range(5) for d in range(5)}
    assert len(classes) == g["classes_lmax4"]
    assert oracle.ncart(4) ** 4 / oracle.nsph(4) ** 4 == pytest.approx(g["spherical_compression_l4"], abs=5e-4)
    # round trip of the class id
    for cid in range(120):
        la, lb, lc, ld = oplan.class_ls(cid)
        assert oplan.class_id(oplan.pair_class(la, lb), oplan.pair_class(lc, ld)) == cid


def test_plan_c1_all_unique():
    g = _golden("structure.txt")
    w = make_config(1)
    sh = w.shells
    S = oracle.schwarz(sh, False)
    p = oplan.screened_plan(sh.l, sh.nprim, S, 0.0)
    assert len(p["index_map"]) == g["unique_quartets_8_shells"]
    seen = set()
    for a, b, c, d, perm in p["index_map"]:
        assert sh.l[a] >= sh.l[b] and sh.l[c] >= sh.l[d]
        assert oplan.pair_class(sh.l[a], sh.l[b]) >= oplan.pair_class(sh.l[c], sh.l[d])
        key = frozenset([frozenset([a, b]), frozenset([c, d])]) if {a, b} != {c, d} else frozenset([frozenset([a, b])])
        assert key not in seen
        seen.add(key)
    assert len({c for c, _, _ in p["blocks"]}) == 6


def test_screened_plan_matches_brute_force():
    """Survivors and order checked against a direct enumeration of all pairs of pairs."""
    w = make_config(3, scale={"natoms": 3})
    sh = w.shells
    S = oracle.schwarz(sh, True)
    tau = 1e-3
    p = oplan.screened_plan(sh.l, sh.nprim, S, tau)
    ns = sh.nshell
    pairs = [(i, j) for i in range(ns) for j in range(i + 1)]
    expect = set()
    for x in range(len(pairs)):
        for y in range(x + 1):
            if S[x] * S[y] >= tau * tau:
                expect.add((x, y))
    got = set()
    for bra, ket in zip(p["pair_bra"], p["pair_ket"]):
        got.add((max(bra, ket), min(bra, ket)))
    assert got == expect
    assert len(got) < len(pairs) * (len(pairs) + 1) // 2  # the screen removed something
    keys = [(c, sh.nprim[a] * sh.nprim[b], sh.nprim[cc] * sh.nprim[d], p["rank"][pb], p["rank"][pk])
            for c, (a, b, cc, d, _), pb, pk in zip(p["class"], p["index_map"], p["pair_bra"], p["pair_ket"])]
    assert keys == sorted(keys)
