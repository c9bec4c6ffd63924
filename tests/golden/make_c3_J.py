"""Write c3_J_spherical.npz: the Coulomb matrix of the 30-atom SVP-like cluster
(seed 1003, spherical, tau = 1e-12, D = C C^T as the workload draws it),
computed by the oracle alone.

Steps: the oracle's Schwarz factors (oracle.schwarz), the oracle's screened
plan of unique quartets (oracle.plan.screened_plan), the oracle's integrals of
every surviving quartet (oracle.eri, four-index Obara-Saika) and the
unique-quartet digestion with the 8-fold symmetry factors
(oracle.J_from_quartets), in chunks whose J are added (the digestion is linear
in the quartets).  J_mu,nu = sum (mu nu|la si) D_la,si is the J update of
Algorithm 2 of "FusionRCG: Orchestrating Recursive Computation Graphs
across GPU Memory Hierarchies".  About 20 minutes on 8 cores.

Usage: python tests/golden/make_c3_J.py
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from oracle import plan as oplan  # noqa: E402
from workloads import make_config  # noqa: E402


def main():
    w = make_config(3)
    sh = w.shells
    t0 = time.time()
    S = oracle.schwarz(sh, True)
    p = oplan.screened_plan(sh.l, sh.nprim, S, w.tau)
    q = np.ascontiguousarray(p["index_map"][:, :4])
    n = sh.nbf(True)
    J = np.zeros((n, n))
    step = 200_000
    for c in range(0, len(q), step):
        sel = q[c:c + step]
        flat, off = oracle.eri(sh, sel, True)
        J += oracle.J_from_quartets(sh, True, sel, flat, off, w.density)
        print(f"{min(c + step, len(q))} / {len(q)} quartets, {time.time() - t0:.0f} s", flush=True)
    np.savez_compressed(os.path.join(HERE, "c3_J_spherical.npz"), J=J, n_quartets=len(q),
                        oracle_threads=oracle.num_threads())
    print(f"wrote c3_J_spherical.npz: {len(q)} quartets, {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
