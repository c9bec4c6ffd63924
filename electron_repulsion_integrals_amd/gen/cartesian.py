"""Cartesian component bookkeeping and the Cartesian-to-spherical coefficients.

Conventions (documented in include/eri.h):
  * Cartesian components of angular momentum l are ordered x-power descending,
    then y-power descending (d: xx, xy, xz, yy, yz, zz).
  * Spherical components are real solid harmonics without Condon-Shortley
    phase, ordered m = -l..l, normalised for the Cartesian shell convention
    used by the library (every Cartesian component of a primitive carries the
    factor that normalises its x^l component).

The coefficients t^(l) of "FusionRCG" section III-B Eq. (8) are not printed on
the page.  Here they are derived from the standard recursion of the real
regular solid harmonics (raise l at m = +-l from x S_ll and y S_l,-l; raise l at
fixed m from z S_lm and r^2 S_l-1,m), then each row is scaled to unit norm
against the Cartesian overlap matrix of the shell and its leading monomial
made positive.
"""
from __future__ import annotations

import math
from functools import lru_cache


def ncart(l: int) -> int:
    return (l + 1) * (l + 2) // 2


def nsph(l: int) -> int:
    return 2 * l + 1


@lru_cache(maxsize=None)
def components(l: int):
    """Cartesian exponent triples of total l in library order."""
    return tuple((i, j, l - i - j) for i in range(l, -1, -1) for j in range(l - i, -1, -1))


@lru_cache(maxsize=None)
def components_upto(L: int):
    """All triples with total <= L, ordered by total then library order."""
    out = []
    for l in range(L + 1):
        out.extend(components(l))
    return tuple(out)


def comp_index(t) -> int:
    """Index of a triple inside its own shell."""
    return components(sum(t)).index(tuple(t))


def sub(t, axis, k=1):
    r = list(t)
    r[axis] -= k
    return tuple(r)


def add(t, axis, k=1):
    r = list(t)
    r[axis] += k
    return tuple(r)


def _poly_mul_xyz(p, axis, scale=1.0):
    out = {}
    for mono, c in p.items():
        m = list(mono)
        m[axis] += 1
        m = tuple(m)
        out[m] = out.get(m, 0.0) + c * scale
    return out


def _poly_add(p, q, sq=1.0):
    out = dict(p)
    for mono, c in q.items():
        out[mono] = out.get(mono, 0.0) + sq * c
    return out


def _poly_scale(p, s):
    return {k: v * s for k, v in p.items()}


def _poly_r2(p):
    out = {}
    for ax in range(3):
        for mono, c in p.items():
            m = list(mono)
            m[ax] += 2
            m = tuple(m)
            out[m] = out.get(m, 0.0) + c
    return out


@lru_cache(maxsize=None)
def _solid_harmonics(lmax: int):
    """S[l][m] as monomial->coefficient dicts, by recursion in l."""
    S = [{0: {(0, 0, 0): 1.0}}]
    for l in range(lmax):
        cur = S[l]
        nxt = {}
        f = math.sqrt((2.0 if l == 0 else 1.0) * (2 * l + 1) / (2 * l + 2))
        # m = l+1 and m = -(l+1)
        xs = _poly_mul_xyz(cur[l], 0)
        ys = _poly_mul_xyz(cur[l], 1)
        if l > 0:
            xs = _poly_add(xs, _poly_mul_xyz(cur[-l], 1), -1.0)
            ys = _poly_add(ys, _poly_mul_xyz(cur[-l], 0), 1.0)
        nxt[l + 1] = _poly_scale(xs, f)
        nxt[-(l + 1)] = _poly_scale(ys, f)
        for m in range(-l, l + 1):
            t = _poly_scale(_poly_mul_xyz(cur[m], 2), 2 * l + 1)
            if abs(m) <= l - 1:
                t = _poly_add(t, _poly_r2(S[l - 1][m]), -math.sqrt((l + m) * (l - m)))
            nxt[m] = _poly_scale(t, 1.0 / math.sqrt((l + m + 1) * (l - m + 1)))
        S.append(nxt)
    return S


def _dfact(n):
    r = 1
    while n > 1:
        r *= n
        n -= 2
    return r


def _overlap(p, q, l):
    s = [p[i] + q[i] for i in range(3)]
    if any(x % 2 for x in s):
        return 0.0
    return _dfact(s[0] - 1) * _dfact(s[1] - 1) * _dfact(s[2] - 1) / _dfact(2 * l - 1)


@lru_cache(maxsize=None)
def sph_matrix(l: int):
    """t^(l) as a tuple of rows (m = -l..l), each a tuple over Cartesian components."""
    S = _solid_harmonics(max(l, 1))[l]
    comps = components(l)
    rows = []
    for m in range(-l, l + 1):
        poly = S[m]
        row = [poly.get(c, 0.0) for c in comps]
        nrm = sum(row[i] * row[j] * _overlap(comps[i], comps[j], l)
                  for i in range(len(comps)) for j in range(len(comps)))
        row = [x / math.sqrt(nrm) for x in row]
        # leading monomial positive: z^l (m=0), x^|m| z^(l-|m|) (m>0), x^(|m|-1) y z^(l-|m|) (m<0)
        am = abs(m)
        lead = (am, 0, l - am) if m > 0 else ((am - 1, 1, l - am) if m < 0 else (0, 0, l))
        if row[comps.index(lead)] < 0:
            row = [-x for x in row]
        rows.append(tuple(0.0 if abs(x) < 1e-15 else x for x in row))
    return tuple(rows)
