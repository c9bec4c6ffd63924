"""Seeded generators for the five benchmark workloads and for smaller test variants.

Recipe (numpy ``Generator(PCG64(seed))``; draw order is part of the recipe):

1. centres (atoms by sequential rejection sampling, or one centre per shell);
2. per shell, in atom-major then l-ascending order: contraction degree K
   (when drawn), then K exponents (log-uniform, i.e. exp(U(ln lo, ln hi))),
   then K contraction coefficients (uniform);
3. for cluster workloads, the matrix C (N x N//4, standard normal) whose
   product C C^T is the density D.

Shells are returned as plain structure-of-arrays:
``centers[S,3]`` (bohr), ``l[S]``, ``nprim[S]``, ``prim_off[S+1]`` (CSR into
``exps``/``coefs``), ``exps``, ``coefs`` (raw, un-normalised coefficients).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

CONFIG_SEEDS = {1: 1001, 2: 1002, 3: 1003, 4: 1004, 5: 1005}

N_SPH = {0: 1, 1: 3, 2: 5, 3: 7, 4: 9}
N_CART = {0: 1, 1: 3, 2: 6, 3: 10, 4: 15}


@dataclass
class ShellSet:
    centers: np.ndarray  # float64 [S,3]
    l: np.ndarray  # int32 [S]
    nprim: np.ndarray  # int32 [S]
    prim_off: np.ndarray  # int32 [S+1]
    exps: np.ndarray  # float64 [sum K]
    coefs: np.ndarray  # float64 [sum K]

    @property
    def nshell(self) -> int:
        return int(self.l.shape[0])

    def nbf(self, spherical: bool) -> int:
        table = N_SPH if spherical else N_CART
        return int(sum(table[int(x)] for x in self.l))


@dataclass
class Workload:
    name: str
    shells: ShellSet
    spherical: bool
    quartets: Optional[np.ndarray]  # int32 [nq,4] explicit list, or None = all unique
    tau: float  # Schwarz threshold (0 = no screening)
    density: Optional[np.ndarray] = None  # float64 [N,N] symmetric PSD
    meta: dict = field(default_factory=dict)


def _loguniform(rng, lo, hi, n):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), n))


def _pack(centers, ls, ks, exps_list, coefs_list) -> ShellSet:
    ks = np.asarray(ks, dtype=np.int32)
    off = np.zeros(len(ks) + 1, dtype=np.int32)
    off[1:] = np.cumsum(ks)
    return ShellSet(
        centers=np.ascontiguousarray(np.asarray(centers, dtype=np.float64).reshape(-1, 3)),
        l=np.asarray(ls, dtype=np.int32),
        nprim=ks,
        prim_off=off,
        exps=np.concatenate(exps_list).astype(np.float64) if exps_list else np.zeros(0),
        coefs=np.concatenate(coefs_list).astype(np.float64) if coefs_list else np.zeros(0),
    )


def _place_atoms(rng, natoms, box, min_sep, max_tries=1_000_000):
    """Sequential rejection sampling of atom positions in [0, box)^3."""
    atoms = []
    tries = 0
    while len(atoms) < natoms:
        tries += 1
        if tries > max_tries:
            raise RuntimeError("could not place atoms with the requested separation")
        cand = rng.uniform(0.0, box, 3)
        if all(np.linalg.norm(cand - a) >= min_sep for a in atoms):
            atoms.append(cand)
    return np.array(atoms)


def cluster(seed: int, natoms: int, box: float, shells_per_l: Sequence[int], kmin: int, kmax: int,
            exp_lo: float, exp_hi: float, coef_lo=0.1, coef_hi=1.0, min_sep=2.0):
    """Atoms placed by rejection sampling; per atom ``shells_per_l[l]`` shells of each l.

    Returns (ShellSet, rng) so callers can continue the draw sequence (density matrix).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    atoms = _place_atoms(rng, natoms, box, min_sep)
    centers, ls, ks, ex, co = [], [], [], [], []
    for a in range(natoms):
        for l, count in enumerate(shells_per_l):
            for _ in range(count):
                k = int(rng.integers(kmin, kmax + 1))
                ex.append(_loguniform(rng, exp_lo, exp_hi, k))
                co.append(rng.uniform(coef_lo, coef_hi, k))
                centers.append(atoms[a])
                ls.append(l)
                ks.append(k)
    return _pack(centers, ls, ks, ex, co), rng


def class_batch(seed: int, ls: Sequence[int], nquartets: int, k: int, box: float,
                exp_lo: float, exp_hi: float, coef_range=(0.1, 1.0), rng=None):
    """``nquartets`` shell quartets of one angular-momentum class, 4 independent centres each.

    Shell 4q+t has angular momentum ls[t].  ``coef_range=None`` means uncontracted
    primitives with coefficient 1.  Returns (ShellSet, quartets[nq,4]).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    nsh = 4 * nquartets
    centers = rng.uniform(0.0, box, (nsh, 3))
    lsh = np.tile(np.asarray(ls, dtype=np.int32), nquartets)
    ex, co = [], []
    for _ in range(nsh):
        ex.append(_loguniform(rng, exp_lo, exp_hi, k))
        if coef_range is None:
            co.append(np.ones(k))
        else:
            co.append(rng.uniform(coef_range[0], coef_range[1], k))
    sh = _pack(centers, lsh, [k] * nsh, ex, co)
    q = np.arange(nsh, dtype=np.int32).reshape(nquartets, 4)
    return sh, q


def random_psd_density(rng, n: int) -> np.ndarray:
    """D = C C^T with C of shape n x (n//4) drawn from N(0,1)."""
    c = rng.standard_normal((n, max(1, n // 4)))
    d = c @ c.T
    return 0.5 * (d + d.T)


def concat_shells(parts: Sequence[ShellSet]) -> ShellSet:
    centers = np.concatenate([p.centers for p in parts])
    ls = np.concatenate([p.l for p in parts])
    ks = np.concatenate([p.nprim for p in parts])
    ex = [p.exps for p in parts]
    co = [p.coefs for p in parts]
    return _pack(centers, ls, ks, ex, co)


def subset_shells(sh: ShellSet, idx: Sequence[int]) -> ShellSet:
    """The shells ``idx`` (in that order) as a new ShellSet."""
    idx = [int(i) for i in idx]
    ex = [sh.exps[sh.prim_off[i]:sh.prim_off[i + 1]] for i in idx]
    co = [sh.coefs[sh.prim_off[i]:sh.prim_off[i + 1]] for i in idx]
    return _pack(sh.centers[idx], sh.l[idx], sh.nprim[idx], ex, co)


def make_config(k: int, scale: Optional[dict] = None) -> Workload:
    """Workload ``k`` (1..5).  ``scale`` shrinks a workload for quick tests.

    scale keys: ``nquartets`` (configs 2 and 4: per-class counts), ``natoms``
    (configs 3 and 5).
    """
    scale = scale or {}
    seed = CONFIG_SEEDS[k]
    if k == 1:
        rng = np.random.Generator(np.random.PCG64(seed))
        atoms = rng.uniform(0.0, 8.0, (4, 3))
        centers, ls, ks, ex, co = [], [], [], [], []
        for a in range(4):
            for l in (0, 1):
                ex.append(_loguniform(rng, 0.1, 50.0, 3))
                co.append(rng.uniform(0.1, 1.0, 3))
                centers.append(atoms[a])
                ls.append(l)
                ks.append(3)
        sh = _pack(centers, ls, ks, ex, co)
        return Workload("tiny s/p molecule, 4 centres, K=3, Cartesian", sh, False, None, 0.0,
                        meta={"seed": seed})
    if k == 2:
        nq = int(scale.get("nquartets", 20000))
        sh, q = class_batch(seed, (2, 2, 2, 2), nq, 1, 10.0, 0.05, 20.0, coef_range=None)
        return Workload(f"(dd|dd) x {nq}, K=1, spherical", sh, True, q, 0.0,
                        meta={"seed": seed, "classes": {"dddd": nq}})
    if k == 4:
        nf = int(scale.get("nquartets_f", scale.get("nquartets", 4000)))
        ng = int(scale.get("nquartets_g", scale.get("nquartets", 4000) // 4 if "nquartets" in scale else 1000))
        rng = np.random.Generator(np.random.PCG64(seed))
        # centres for all shells first, then per-shell primitives (draw order of the recipe)
        nsh = 4 * (nf + ng)
        centers = rng.uniform(0.0, 10.0, (nsh, 3))
        ls = np.array([3] * (4 * nf) + [4] * (4 * ng), dtype=np.int32)
        ex, co = [], []
        for _ in range(nsh):
            ex.append(_loguniform(rng, 0.1, 10.0, 2))
            co.append(rng.uniform(0.1, 1.0, 2))
        sh = _pack(centers, ls, [2] * nsh, ex, co)
        q = np.arange(nsh, dtype=np.int32).reshape(-1, 4)
        return Workload(f"(ff|ff) x {nf} + (gg|gg) x {ng}, K=2, spherical", sh, True, q, 0.0,
                        meta={"seed": seed, "classes": {"ffff": nf, "gggg": ng}})
    if k == 3:
        natoms = int(scale.get("natoms", 30))
        sh, rng = cluster(seed, natoms, 20.0, (3, 2, 1), 1, 6, 0.1, 5000.0)
        n = sh.nbf(True)
        d = random_psd_density(rng, n)
        return Workload(f"{natoms}-atom SVP-like cluster, tau=1e-12, spherical J", sh, True, None, 1e-12,
                        density=d, meta={"seed": seed, "natoms": natoms, "nbf": n})
    if k == 5:
        natoms = int(scale.get("natoms", 120))
        sh, rng = cluster(seed, natoms, 35.0, (5, 4, 3, 1), 1, 8, 0.05, 1e4)
        n = sh.nbf(True)
        d = random_psd_density(rng, n)
        return Workload(f"{natoms}-atom TZVP-like cluster, tau=1e-12, spherical J", sh, True, None, 1e-12,
                        density=d, meta={"seed": seed, "natoms": natoms, "nbf": n})
    raise ValueError(f"unknown config {k}")
