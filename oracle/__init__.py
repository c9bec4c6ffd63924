"""CPU oracle for the ERI engine -- TEST INFRASTRUCTURE ONLY.

Plain, slow fp64 reference implementations written from "FusionRCG:
Orchestrating Recursive Computation Graphs across GPU Memory Hierarchies"
(section II-A Eq. (1)-(3), section III-B Eq. (8) and (17), section III-C
Algorithm 2).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and never calls it.

Parts:
  * ``eri_oracle.c`` (C, OpenMP): Boys function, normalisation, spherical
    coefficients, four-index Obara-Saika integrals, Schwarz factors, J.
  * ``plan.py`` (numpy): the quartet plan -- canonical class form, sort key,
    Schwarz screening -- written out as plainly as possible.

The C source builds twice: ``liberi_oracle.so`` computes in fp64 (the oracle
every test compares against), ``liberi_oracle_q.so`` compiles the same source
with IEEE binary128 arithmetic (``-DORACLE_QUAD``).  The second exists only to
adjudicate: it measures how far the fp64 oracle is from the exact value of the
same definition (``precision="quad"`` on the functions below).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "eri_oracle.c")
LIB = os.path.join(HERE, "liberi_oracle.so")
QLIB = os.path.join(HERE, "liberi_oracle_q.so")
_GCC = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC"]
# Tests that plant a mistake in the oracle point this at a mutant build.
_LIB_OVERRIDE = os.environ.get("ERI_ORACLE_LIB")

SPHERICAL = 1
NO_NORMALIZE = 2


def build(force: bool = False, out: str = None, defines=()) -> str:
    """Compile the C oracle with gcc (always when ``force`` or ``out`` is given):
    the fp64 library, and with ``force`` also the binary128 adjudication build."""
    if out is not None:
        subprocess.check_call([*_GCC, *[f"-D{d}" for d in defines], "-o", out, SRC, "-lm"])
        return out
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call([*_GCC, "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    if force:
        build_quad(force=True)
    return LIB


def build_quad(force: bool = False) -> str:
    """Compile the binary128 adjudication build of the same source."""
    if force or not os.path.exists(QLIB) or os.path.getmtime(QLIB) < os.path.getmtime(SRC):
        tmp = QLIB + ".tmp"
        subprocess.check_call([*_GCC, "-DORACLE_QUAD", "-o", tmp, SRC, "-lquadmath", "-lm"])
        os.replace(tmp, QLIB)
    return QLIB


_lib = None
_qlib = None


def lib(precision: str = "fp64"):
    """The fp64 oracle library, or with precision="quad" its binary128 build."""
    global _lib, _qlib
    if precision == "quad":
        if _qlib is None:
            _qlib = _bind(ctypes.CDLL(build_quad()))
        return _qlib
    if precision != "fp64":
        raise ValueError(precision)
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(LIB)
        _lib = _bind(L)
    return _lib


def _bind(L):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lp = ctypes.POINTER(ctypes.c_int64)
    L.oracle_boys.argtypes = [ctypes.c_int, ctypes.c_double, dp]
    L.oracle_boys.restype = None
    L.oracle_normalize.argtypes = [ctypes.c_int, ctypes.c_int, dp, dp, dp]
    L.oracle_sph_coeffs.argtypes = [ctypes.c_int, dp]
    L.oracle_eri_quartets.argtypes = [ctypes.c_int, dp, ip, ip, ip, dp, dp, ctypes.c_int,
                                      ctypes.c_int64, ip, lp, dp]
    L.oracle_eri_quartets.restype = ctypes.c_int
    L.oracle_eri_deriv_quartets.argtypes = [ctypes.c_int, dp, ip, ip, ip, dp, dp, ctypes.c_int,
                                            ctypes.c_int64, ip, lp, dp]
    L.oracle_eri_deriv_quartets.restype = ctypes.c_int
    L.oracle_schwarz.argtypes = [ctypes.c_int, dp, ip, ip, ip, dp, dp, ctypes.c_int, dp]
    L.oracle_schwarz.restype = ctypes.c_int
    L.oracle_J_from_quartets.argtypes = [ctypes.c_int, ip, ctypes.c_int, ip, ctypes.c_int,
                                         ctypes.c_int64, ip, lp, dp, dp, dp]
    L.oracle_J_from_quartets.restype = None
    L.oracle_J_naive.argtypes = [ctypes.c_int, dp, ip, ip, ip, dp, dp, ctypes.c_int, ip,
                                 ctypes.c_int, dp, dp]
    L.oracle_J_naive.restype = ctypes.c_int
    L.oracle_K_from_quartets.argtypes = [ctypes.c_int, ip, ctypes.c_int, ip, ctypes.c_int,
                                         ctypes.c_int64, ip, lp, dp, dp, dp]
    L.oracle_K_from_quartets.restype = None
    L.oracle_K_naive.argtypes = [ctypes.c_int, dp, ip, ip, ip, dp, dp, ctypes.c_int, ip,
                                 ctypes.c_int, dp, dp]
    L.oracle_K_naive.restype = ctypes.c_int
    L.oracle_num_threads.restype = ctypes.c_int
    return L


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _i(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _l(a):
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def ncart(l):
    return (l + 1) * (l + 2) // 2


def nsph(l):
    return 2 * l + 1


def nfunc(l, spherical):
    return nsph(l) if spherical else ncart(l)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def boys(mmax: int, T: float, precision: str = "fp64") -> np.ndarray:
    """F_0..F_mmax at T (series + downward recursion, or erf + upward above T=50)."""
    out = np.zeros(mmax + 1)
    out_, p = _d(out)
    lib(precision).oracle_boys(int(mmax), float(T), p)
    return out_


def normalize(l: int, exps, coefs) -> np.ndarray:
    e, pe = _d(exps)
    c, pc = _d(coefs)
    out = np.zeros_like(e)
    o, po = _d(out)
    lib().oracle_normalize(int(l), len(e), pe, pc, po)
    return o


def sph_coeffs(l: int) -> np.ndarray:
    """T^(l) of Eq. (8): (2l+1) x ncart(l), rows m = -l..l, columns in Cartesian order."""
    out = np.zeros((nsph(l), ncart(l)))
    o, p = _d(out)
    lib().oracle_sph_coeffs(int(l), p)
    return o


def cart_components(l: int):
    return [(i, j, l - i - j) for i in range(l, -1, -1) for j in range(l - i, -1, -1)]


def _shell_args(sh):
    c, pc = _d(sh.centers)
    l, pl = _i(sh.l)
    k, pk = _i(sh.nprim)
    o, po = _i(sh.prim_off)
    e, pe = _d(sh.exps)
    cf, pcf = _d(sh.coefs)
    keep = (c, l, k, o, e, cf)
    return keep, (int(sh.l.shape[0]), pc, pl, pk, po, pe, pcf)


def block_sizes(sh, quartets, spherical):
    q = np.asarray(quartets, dtype=np.int64).reshape(-1, 4)
    n = np.array([nfunc(int(x), spherical) for x in sh.l], dtype=np.int64)
    return n[q[:, 0]] * n[q[:, 1]] * n[q[:, 2]] * n[q[:, 3]]


def eri(sh, quartets, spherical: bool, normalize_: bool = True, precision: str = "fp64"):
    """Integral blocks for each quartet (shell order as given).

    Returns (flat values, offsets[nq]) with block q at flat[off[q]: off[q]+size[q]],
    row-major over (a, b, c, d).  precision="quad" evaluates the same definition
    in binary128 and rounds the results to fp64 (adjudication only).
    """
    q, pq = _i(np.asarray(quartets).reshape(-1, 4))
    sizes = block_sizes(sh, q, spherical)
    off = np.zeros(len(sizes), dtype=np.int64)
    if len(sizes) > 1:
        off[1:] = np.cumsum(sizes)[:-1]
    out = np.zeros(int(sizes.sum()) if len(sizes) else 0)
    o, po = _d(out)
    of, pof = _l(off)
    keep, args = _shell_args(sh)
    flags = (SPHERICAL if spherical else 0) | (0 if normalize_ else NO_NORMALIZE)
    rc = lib(precision).oracle_eri_quartets(*args, flags, len(q), pq, pof, po)
    if rc != 0:
        raise ValueError("oracle_eri_quartets rejected its input")
    return o, of


def eri_deriv(sh, quartets, spherical: bool, normalize_: bool = True):
    """First derivatives of each quartet's block with respect to the centres of
    its four shells (in the order given): 12 blocks per quartet, in the order
    d/dA_x, d/dA_y, d/dA_z, d/dB_x, ..., d/dD_z, each row-major over (a, b, c, d).

    Returns (flat values, offsets[nq]); quartet q's 12 blocks start at off[q].
    Differentiating a Cartesian Gaussian with respect to its own centre raises
    and lowers its angular momentum: d/dA_i phi_a = 2 alpha phi_(a+1_i) - a_i phi_(a-1_i).
    """
    q, pq = _i(np.asarray(quartets).reshape(-1, 4))
    sizes = 12 * block_sizes(sh, q, spherical)
    off = np.zeros(len(sizes), dtype=np.int64)
    if len(sizes) > 1:
        off[1:] = np.cumsum(sizes)[:-1]
    out = np.zeros(int(sizes.sum()) if len(sizes) else 0)
    o, po = _d(out)
    of, pof = _l(off)
    keep, args = _shell_args(sh)
    flags = (SPHERICAL if spherical else 0) | (0 if normalize_ else NO_NORMALIZE)
    rc = lib().oracle_eri_deriv_quartets(*args, flags, len(q), pq, pof, po)
    if rc != 0:
        raise ValueError("oracle_eri_deriv_quartets rejected its input")
    return o, of


def eri_deriv_block(sh, quartet, spherical: bool, normalize_: bool = True) -> np.ndarray:
    """One quartet's derivatives as an array [4 centres, 3 axes, a, b, c, d]."""
    flat, _ = eri_deriv(sh, [quartet], spherical, normalize_)
    dims = [nfunc(int(sh.l[s]), spherical) for s in quartet]
    return flat.reshape([4, 3] + dims)


def eri_block(sh, quartet, spherical: bool, normalize_: bool = True, precision: str = "fp64") -> np.ndarray:
    """One quartet as a 4-index array."""
    flat, _ = eri(sh, [quartet], spherical, normalize_, precision)
    dims = [nfunc(int(sh.l[s]), spherical) for s in quartet]
    return flat.reshape(dims)


def schwarz(sh, spherical: bool, precision: str = "fp64") -> np.ndarray:
    """S[p] for pairs i >= j, p = i(i+1)/2 + j."""
    ns = int(sh.l.shape[0])
    out = np.zeros(ns * (ns + 1) // 2)
    o, po = _d(out)
    keep, args = _shell_args(sh)
    rc = lib(precision).oracle_schwarz(*args, SPHERICAL if spherical else 0, po)
    if rc != 0:
        raise ValueError("oracle_schwarz failed")
    return o


def basis_offsets(sh, spherical: bool) -> np.ndarray:
    n = np.array([nfunc(int(x), spherical) for x in sh.l], dtype=np.int32)
    off = np.zeros(len(n) + 1, dtype=np.int32)
    off[1:] = np.cumsum(n)
    return off


def J_from_quartets(sh, spherical: bool, quartets, flat, off, D) -> np.ndarray:
    """J from unique quartets with the per-pair factor-2 rule (see eri_oracle.c)."""
    bf = basis_offsets(sh, spherical)
    nbf = int(bf[-1])
    q, pq = _i(np.asarray(quartets).reshape(-1, 4))
    l, pl = _i(sh.l)
    b, pb = _i(bf)
    f, pf = _d(flat)
    of, pof = _l(off)
    d, pd = _d(D)
    J = np.zeros((nbf, nbf))
    j, pj = _d(J)
    lib().oracle_J_from_quartets(int(sh.l.shape[0]), pl, SPHERICAL if spherical else 0, pb, nbf,
                                 len(q), pq, pof, pf, pd, pj)
    return j


def J_naive(sh, spherical: bool, D) -> np.ndarray:
    """J by the plain sum over every ordered shell quadruple (tiny inputs only)."""
    bf = basis_offsets(sh, spherical)
    nbf = int(bf[-1])
    b, pb = _i(bf)
    d, pd = _d(D)
    J = np.zeros((nbf, nbf))
    j, pj = _d(J)
    keep, args = _shell_args(sh)
    rc = lib().oracle_J_naive(*args, SPHERICAL if spherical else 0, pb, nbf, pd, pj)
    if rc != 0:
        raise ValueError("oracle_J_naive failed")
    return j


def K_from_quartets(sh, spherical: bool, quartets, flat, off, D) -> np.ndarray:
    """K_mu,nu = sum (mu la|nu si) D_la,si from unique quartets: every distinct
    index permutation of each quartet added once (see eri_oracle.c)."""
    bf = basis_offsets(sh, spherical)
    nbf = int(bf[-1])
    q, pq = _i(np.asarray(quartets).reshape(-1, 4))
    l, pl = _i(sh.l)
    b, pb = _i(bf)
    f, pf = _d(flat)
    of, pof = _l(off)
    d, pd = _d(D)
    K = np.zeros((nbf, nbf))
    k, pk = _d(K)
    lib().oracle_K_from_quartets(int(sh.l.shape[0]), pl, SPHERICAL if spherical else 0, pb, nbf,
                                 len(q), pq, pof, pf, pd, pk)
    return k


def K_naive(sh, spherical: bool, D) -> np.ndarray:
    """K by the plain sum over every ordered shell quadruple (tiny inputs only)."""
    bf = basis_offsets(sh, spherical)
    nbf = int(bf[-1])
    b, pb = _i(bf)
    d, pd = _d(D)
    K = np.zeros((nbf, nbf))
    k, pk = _d(K)
    keep, args = _shell_args(sh)
    rc = lib().oracle_K_naive(*args, SPHERICAL if spherical else 0, pb, nbf, pd, pk)
    if rc != 0:
        raise ValueError("oracle_K_naive failed")
    return k


def J_blocks(sh, spherical: bool, bra_pairs, D, S, tau):
    """J blocks for the given shell pairs (i, j) by the plain sum over every ket pair.

    J_mu,nu = sum over shell pairs (k >= l) of f_kl sum_(la in k, si in l) (mu nu|la si) D_la,si,
    f_kl = 2 for k != l (the (l, k) orientation of a symmetric D), keeping only the
    pairs with fl(S_ij * S_kl) >= fl(tau^2) (S indexed by pair index i(i+1)/2 + j).
    Returns a list of arrays [n_i, n_j].
    """
    ns = int(sh.l.shape[0])
    bf = basis_offsets(sh, spherical)
    t2 = float(tau) * float(tau)
    out = []
    kets = [(k, l) for k in range(ns) for l in range(k + 1)]
    for (i, j) in bra_pairs:
        pij = max(i, j) * (max(i, j) + 1) // 2 + min(i, j)
        keep = [(k, l) for (k, l) in kets if S[pij] * S[k * (k + 1) // 2 + l] >= t2]
        q = [(i, j, k, l) for (k, l) in keep]
        flat, off = eri(sh, q, spherical)
        ni, nj = nfunc(int(sh.l[i]), spherical), nfunc(int(sh.l[j]), spherical)
        J = np.zeros((ni, nj))
        for t, (k, l) in enumerate(keep):
            nk, nl = nfunc(int(sh.l[k]), spherical), nfunc(int(sh.l[l]), spherical)
            blk = flat[off[t]: off[t] + ni * nj * nk * nl].reshape(ni, nj, nk, nl)
            f = 2.0 if k != l else 1.0
            J += f * np.einsum("abcd,cd->ab", blk, D[bf[k]:bf[k + 1], bf[l]:bf[l + 1]])
        out.append(J)
    return out


def K_blocks(sh, spherical: bool, pairs, D, S, tau):
    """K blocks for the given ordered shell pairs (i, k) by the plain sum
    K_mu,nu = sum over every shell j and every shell l of
    sum_(la in j, si in l) (mu la|nu si) D_la,si, keeping only the quartets with
    fl(S_ij * S_kl) >= fl(tau^2) (S indexed by pair index).  Returns a list of
    arrays [n_i, n_k]."""
    ns = int(sh.l.shape[0])
    bf = basis_offsets(sh, spherical)
    t2 = float(tau) * float(tau)

    def pidx(x, y):
        return max(x, y) * (max(x, y) + 1) // 2 + min(x, y)
    out = []
    for (i, k) in pairs:
        keep = [(j, l) for j in range(ns) for l in range(ns) if S[pidx(i, j)] * S[pidx(k, l)] >= t2]
        q = [(i, j, k, l) for (j, l) in keep]
        flat, off = eri(sh, q, spherical)
        ni, nk = nfunc(int(sh.l[i]), spherical), nfunc(int(sh.l[k]), spherical)
        K = np.zeros((ni, nk))
        for t, (j, l) in enumerate(keep):
            nj, nl = nfunc(int(sh.l[j]), spherical), nfunc(int(sh.l[l]), spherical)
            blk = flat[off[t]: off[t] + ni * nj * nk * nl].reshape(ni, nj, nk, nl)
            K += np.einsum("abcd,bd->ac", blk, D[bf[j]:bf[j + 1], bf[l]:bf[l + 1]])
        out.append(K)
    return out


def _intermediate_magnitudes(sh, a, b, c, d, normalize_: bool, per_primitive: bool):
    """{(e, f): magnitude} of the contracted intermediates [e0|f0] of quartet
    (a b|c d), |e| in [l_a, l_a+l_b], |f| in [l_c, l_c+l_d]: |[e0|f0]|, or with
    per_primitive the sum over the primitive quartets of |their term|."""
    import itertools
    from workloads.configs import _pack
    la, lb, lc, ld = (int(sh.l[s]) for s in (a, b, c, d))
    prim = []
    for s, l in ((a, la), (b, lb), (c, lc), (d, ld)):
        e = sh.exps[sh.prim_off[s]:sh.prim_off[s + 1]]
        raw = sh.coefs[sh.prim_off[s]:sh.prim_off[s + 1]]
        prim.append((np.asarray(e, dtype=float), normalize(l, e, raw) if normalize_ else np.asarray(raw, dtype=float)))
    cen = [sh.centers[s] for s in (a, b, c, d)]
    V = {}
    for le in range(la, la + lb + 1):
        for lf in range(lc, lc + ld + 1):
            if not per_primitive:
                s2 = _pack(cen, [le, 0, lf, 0], [len(p[0]) for p in prim], [p[0] for p in prim], [p[1] for p in prim])
                mag = np.abs(eri_block(s2, [0, 1, 2, 3], False, normalize_=False)[:, 0, :, 0])
            else:
                # one shell per primitive; every primitive quartet as its own quartet
                C, L, E, CF, first = [], [], [], [], []
                for t, ((e, co), l) in enumerate(zip(prim, (le, 0, lf, 0))):
                    first.append(len(L))
                    for x in range(len(e)):
                        C.append(cen[t])
                        L.append(l)
                        E.append(e[x:x + 1])
                        CF.append(co[x:x + 1])
                s2 = _pack(np.array(C), L, [1] * len(L), E, CF)
                qs = [[first[0] + i, first[1] + j, first[2] + k, first[3] + m]
                      for i, j, k, m in itertools.product(*[range(len(p[0])) for p in prim])]
                flat, _ = eri(s2, qs, False, normalize_=False)
                n1, n2 = len(cart_components(le)), len(cart_components(lf))
                mag = np.abs(flat.reshape(len(qs), n1, n2)).sum(axis=0)
            for i, e_ in enumerate(cart_components(le)):
                for j, f_ in enumerate(cart_components(lf)):
                    V[(e_, f_)] = mag[i, j]
    return V


def hgp_rounding_bound(sh, quartets, spherical: bool, eps: float = 2.0 ** -53, normalize_: bool = True,
                       per_primitive: bool = False):
    """First-order fp64 error floor of the two-phase (VRR + HRR) evaluation.

    The two-phase method holds the contracted intermediates
    [e0|f0] = (e_A s_B | f_C s_D), |e| in [l_a, l_a+l_b], |f| in [l_c, l_c+l_d]
    (the exponents and normalised contraction coefficients of the quartet's
    shells), and the horizontal recurrence Eq. (3) expands each target as
        (a b|c d) = sum_k sum_k' prod_i C(b_i,k_i) AB_i^(b_i-k_i) C(d_i,k'_i) CD_i^(d_i-k'_i) [a+k 0|c+k' 0]
    (the recurrence unrolled by the binomial theorem, AB = A - B, CD = C - D).
    Rounding every intermediate to fp64 (relative error eps) therefore moves
    the target by up to  eps * sum |coefficient| |[a+k 0|c+k' 0]|,  which this
    function returns per element (spherical outputs by the triangle inequality
    through |t^(l)|).  It is the error that storing the intermediates in fp64
    alone forces on any such evaluation; for diffuse high-l quartets it can far
    exceed 1e-10 of the result.  The intermediates are computed here by the
    oracle's own four-index recurrence on raw primitives, weighted by the
    normalised contraction coefficients, or by the raw ones with
    normalize_=False (for quartets evaluated with raw coefficients).  With
    per_primitive, |[a+k 0|c+k' 0]| is replaced by the sum over the primitive
    quartets of the magnitudes of their terms (see contraction_rounding_bound).
    """
    from math import comb
    q = np.asarray(quartets).reshape(-1, 4)
    out = []
    for a, b, c, d in q:
        la, lb, lc, ld = (int(sh.l[s]) for s in (a, b, c, d))
        V = _intermediate_magnitudes(sh, a, b, c, d, normalize_, per_primitive)
        AB = np.abs(sh.centers[a] - sh.centers[b])
        CD = np.abs(sh.centers[c] - sh.centers[d])

        def expand(x, y, R):
            """[(coefficient magnitude, x + k)] of the unrolled HRR for (x, y)."""
            terms = [(1.0, (0, 0, 0))]
            for ax in range(3):
                new = []
                for cf, k in terms:
                    for ki in range(y[ax] + 1):
                        kk = list(k)
                        kk[ax] = ki
                        new.append((cf * comb(y[ax], ki) * R[ax] ** (y[ax] - ki), tuple(kk)))
                terms = new
            return [(cf, (x[0] + k[0], x[1] + k[1], x[2] + k[2])) for cf, k in terms]

        ca, cb, cc, cd = (cart_components(l) for l in (la, lb, lc, ld))
        bound = np.zeros((len(ca), len(cb), len(cc), len(cd)))
        for ia, xa in enumerate(ca):
            for ib, yb in enumerate(cb):
                bt = expand(xa, yb, AB)
                for ic, xc in enumerate(cc):
                    for id_, yd in enumerate(cd):
                        kt = expand(xc, yd, CD)
                        bound[ia, ib, ic, id_] = sum(c1 * c2 * V[(e1, f1)] for c1, e1 in bt for c2, f1 in kt)
        bound *= eps
        if spherical:
            for pos, l in enumerate((la, lb, lc, ld)):
                bound = np.moveaxis(np.tensordot(np.abs(sph_coeffs(l)), np.moveaxis(bound, pos, 0), axes=(1, 0)), 0, pos)
        out.append(bound.ravel())
    return np.concatenate(out) if out else np.zeros(0)


def contraction_rounding_bound(sh, quartets, spherical: bool, eps: float = 2.0 ** -53):
    """Floor for the rounding of the contraction sums of the two-phase method.

    Each contracted intermediate [e0|f0] is a sum of K4 = K_a K_b K_c K_d
    primitive terms accumulated in fp64.  The worst-case bound on the rounding
    of such a sum grows as (K4 - 1) eps sum |term|; the probabilistic analysis
    of Higham and Mary ("A new approach to probabilistic rounding error
    analysis", SIAM J. Sci. Comput. 41, 2019) shows that with independent
    rounding errors it grows as lambda sqrt(K4 - 1) eps sum |term|, lambda a
    small constant that sets the confidence.  This returns, per element,
    sqrt(K4 - 1) times hgp_rounding_bound with the per-primitive magnitudes
    (that bound at lambda = 1, propagated through the unrolled horizontal
    recurrence); the caller chooses lambda.  Zero for K4 = 1."""
    q = np.asarray(quartets).reshape(-1, 4)
    out = []
    for row in q:
        k4 = int(np.prod([int(sh.prim_off[s + 1] - sh.prim_off[s]) for s in row]))
        if k4 <= 1:
            out.append(np.zeros(int(block_sizes(sh, row[None, :], spherical)[0])))
            continue
        out.append(np.sqrt(k4 - 1.0) * hgp_rounding_bound(sh, row[None, :], spherical, eps, per_primitive=True))
    return np.concatenate(out) if out else np.zeros(0)


def _unrolled_hrr_abs(la, lb, R):
    """|coefficients| of the horizontal recurrence unrolled by the binomial
    theorem: rows the Cartesian pairs (a, b) of shells la, lb (row-major), columns
    the components e of the intermediates [e0| with |e| = la..la+lb (by |e|, then
    Cartesian order); (a b| = sum_e coefficient x [e 0|, each coefficient a
    product of C(b_i, k_i) |R_i|^(b_i - k_i), R = A - B."""
    from math import comb
    ca, cb = cart_components(la), cart_components(lb)
    cols = {}
    for le in range(la, la + lb + 1):
        for e in cart_components(le):
            cols[e] = len(cols)
    M = np.zeros((len(ca) * len(cb), len(cols)))
    for ia, xa in enumerate(ca):
        for ib, yb in enumerate(cb):
            terms = [(1.0, (0, 0, 0))]
            for ax in range(3):
                terms = [(cf * comb(yb[ax], ki) * abs(R[ax]) ** (yb[ax] - ki),
                          tuple(ki if t == ax else k[t] for t in range(3)))
                         for cf, k in terms for ki in range(yb[ax] + 1)]
            for cf, k in terms:
                M[ia * len(cb) + ib, cols[(xa[0] + k[0], xa[1] + k[1], xa[2] + k[2])]] += cf
    return M


def _oriented(sh, i, j):
    """The pair (i, j) in the order the library evaluates it: the shell of
    higher l first, the higher shell index first when the l are equal."""
    i, j = max(i, j), min(i, j)
    return (j, i) if sh.l[i] < sh.l[j] else (i, j)


def hgp_rounding_bound_J(sh, spherical: bool, bra_pairs, D, S, tau, eps: float = 2.0 ** -53):
    """The two-phase fp64 floor (hgp_rounding_bound) propagated into J blocks.

    For each requested shell pair (i, j), F_ij = sum over the ket pairs (k, l)
    that pass the Schwarz test of f_kl sum_(cd) B(ij|kl)[ab, cd] |D_cd| with
    f_kl = 2 for k != l, B the per-element floor of the quartet in the
    orientation the library evaluates it in (see _oriented).  A J element whose
    integrals each carry an error of at most c x B is off by at most c x F.
    Computed with matrices: B = eps |T| M_bra V M_ket^T |T|^T, M the unrolled
    horizontal recurrences (_unrolled_hrr_abs), V the magnitudes of the oracle's
    contracted intermediates (e_A s_B | f_C s_D), obtained for every ket in one
    batch.  Returns a list of arrays [n_i, n_j] in the requested orientation.
    """
    from workloads.configs import _pack
    ns = int(sh.l.shape[0])
    bf = basis_offsets(sh, spherical)
    LMAX = 9
    # every shell again with l' = 0..8 on raw monomials, normalised coefficients of its own l
    cen, ls, ks, ex, co = [], [], [], [], []
    for s in range(ns):
        e = sh.exps[sh.prim_off[s]:sh.prim_off[s + 1]]
        c = normalize(int(sh.l[s]), e, sh.coefs[sh.prim_off[s]:sh.prim_off[s + 1]])
        for lp in range(LMAX):
            cen.append(sh.centers[s])
            ls.append(lp)
            ks.append(len(e))
            ex.append(e)
            co.append(c)
    aug = _pack(cen, ls, ks, ex, co)
    t2 = float(tau) * float(tau)
    kets = [(k, l) for k in range(ns) for l in range(k + 1)]
    T = [np.abs(sph_coeffs(l)) for l in range(5)]
    out = []
    for (i, j) in bra_pairs:
        a, b = _oriented(sh, i, j)
        la, lb = int(sh.l[a]), int(sh.l[b])
        pij = max(i, j) * (max(i, j) + 1) // 2 + min(i, j)
        keep = [_oriented(sh, k, l) for (k, l) in kets if S[pij] * S[k * (k + 1) // 2 + l] >= t2]
        Mb = _unrolled_hrr_abs(la, lb, sh.centers[a] - sh.centers[b])
        if spherical:
            Mb = np.kron(T[la], T[lb]) @ Mb
        u = np.zeros(Mb.shape[1])
        # intermediates of every kept ket, batched by (l_e, l_f)
        q, where = [], []
        for t, (c, d) in enumerate(keep):
            lc, ld = int(sh.l[c]), int(sh.l[d])
            for le in range(la, la + lb + 1):
                for lf in range(lc, lc + ld + 1):
                    q.append((a * LMAX + le, b * LMAX, c * LMAX + lf, d * LMAX))
                    where.append((t, le, lf))
        flat, off = eri(aug, q, False, normalize_=False)
        ends = np.append(np.asarray(off), len(flat))
        V = {}
        for x, (t, le, lf) in enumerate(where):
            V[(t, le, lf)] = np.abs(flat[ends[x]:ends[x + 1]]).reshape(ncart(le), ncart(lf))
        for t, (c, d) in enumerate(keep):
            lc, ld = int(sh.l[c]), int(sh.l[d])
            Vt = np.block([[V[(t, le, lf)] for lf in range(lc, lc + ld + 1)] for le in range(la, la + lb + 1)])
            Mk = _unrolled_hrr_abs(lc, ld, sh.centers[c] - sh.centers[d])
            if spherical:
                Mk = np.kron(T[lc], T[ld]) @ Mk
            w = Mk.T @ np.abs(D[bf[c]:bf[c + 1], bf[d]:bf[d + 1]]).ravel()
            u += (2.0 if c != d else 1.0) * (Vt @ w)
        F = (eps * (Mb @ u)).reshape(nfunc(la, spherical), nfunc(lb, spherical))
        out.append(F if a == i else F.T)
    return out
