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
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "eri_oracle.c")
LIB = os.path.join(HERE, "liberi_oracle.so")
# Tests that plant a mistake in the oracle point this at a mutant build.
_LIB_OVERRIDE = os.environ.get("ERI_ORACLE_LIB")

SPHERICAL = 1
NO_NORMALIZE = 2


def build(force: bool = False, out: str = None, defines=()) -> str:
    """Compile the C oracle with gcc (always when ``force`` or ``out`` is given)."""
    if out is not None:
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                               *[f"-D{d}" for d in defines], "-o", out, SRC, "-lm"])
        return out
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                               "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(LIB)
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
        L.oracle_schwarz.argtypes = [ctypes.c_int, dp, ip, ip, ip, dp, dp, ctypes.c_int, dp]
        L.oracle_schwarz.restype = ctypes.c_int
        L.oracle_J_from_quartets.argtypes = [ctypes.c_int, ip, ctypes.c_int, ip, ctypes.c_int,
                                             ctypes.c_int64, ip, lp, dp, dp, dp]
        L.oracle_J_from_quartets.restype = None
        L.oracle_J_naive.argtypes = [ctypes.c_int, dp, ip, ip, ip, dp, dp, ctypes.c_int, ip,
                                     ctypes.c_int, dp, dp]
        L.oracle_J_naive.restype = ctypes.c_int
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


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


def boys(mmax: int, T: float) -> np.ndarray:
    """F_0..F_mmax at T (series + downward recursion, or erf + upward above T=50)."""
    out = np.zeros(mmax + 1)
    out_, p = _d(out)
    lib().oracle_boys(int(mmax), float(T), p)
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


def eri(sh, quartets, spherical: bool, normalize_: bool = True):
    """Integral blocks for each quartet (shell order as given).

    Returns (flat values, offsets[nq]) with block q at flat[off[q]: off[q]+size[q]],
    row-major over (a, b, c, d).
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
    rc = lib().oracle_eri_quartets(*args, flags, len(q), pq, pof, po)
    if rc != 0:
        raise ValueError("oracle_eri_quartets rejected its input")
    return o, of


def eri_block(sh, quartet, spherical: bool, normalize_: bool = True) -> np.ndarray:
    """One quartet as a 4-index array."""
    flat, _ = eri(sh, [quartet], spherical, normalize_)
    dims = [nfunc(int(sh.l[s]), spherical) for s in quartet]
    return flat.reshape(dims)


def schwarz(sh, spherical: bool) -> np.ndarray:
    """S[p] for pairs i >= j, p = i(i+1)/2 + j."""
    ns = int(sh.l.shape[0])
    out = np.zeros(ns * (ns + 1) // 2)
    o, po = _d(out)
    keep, args = _shell_args(sh)
    rc = lib().oracle_schwarz(*args, SPHERICAL if spherical else 0, po)
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
