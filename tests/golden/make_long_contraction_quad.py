"""Write long_contraction_quad.npz: one (gf|dd) quartet with contraction
degrees 6, 7, 6, 8 (2,016 primitive quartets; shells drawn with seed 31,
exponents log-uniform in [0.1, 50], centres in a 2.5-bohr cube), its shells,
and its spherical integral block evaluated by the oracle's binary128 build
(oracle.eri_block with precision="quad": the plain four-index Obara-Saika
definition of Eq. (1) of "FusionRCG: Orchestrating Recursive Computation Graphs
across GPU Memory Hierarchies", section II-A, in IEEE binary128, results
rounded to fp64).  About three minutes on one core.

Usage: python tests/golden/make_long_contraction_quad.py
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads.configs import _pack  # noqa: E402

QUARTET = [3, 1, 5, 4]


def shells():
    rng = np.random.default_rng(31)
    ls = [3, 3, 4, 4, 2, 2, 1, 0, 4]
    ks = [6, 7, 6, 8, 8, 6, 7, 8, 5]
    return _pack(rng.uniform(0, 2.5, (len(ls), 3)), ls, ks,
                 [np.exp(rng.uniform(np.log(0.1), np.log(50), k)) for k in ks], [rng.uniform(0.1, 1, k) for k in ks])


def main():
    sh = shells()
    t = time.time()
    x = oracle.eri_block(sh, QUARTET, True, precision="quad").ravel()
    print(f"binary128 block of {len(x)} elements in {time.time() - t:.0f} s")
    np.savez(os.path.join(HERE, "long_contraction_quad.npz"), quartet=np.array(QUARTET), centers=sh.centers,
             l=sh.l, nprim=sh.nprim, prim_off=sh.prim_off, exps=sh.exps, coefs=sh.coefs, quad=x)


if __name__ == "__main__":
    main()
