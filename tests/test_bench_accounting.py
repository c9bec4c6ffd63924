"""bench.py's count of the primitive quartets a screened plan evaluates (its
FP64 accounting) follows the same primitive-pair rule as the oracle's plan
twin: per quartet, the product of the two shell pairs' kept primitive pairs;
for an explicit list, the product of the four contraction degrees."""
import numpy as np

import bench
from oracle import plan as oplan
from workloads import make_config


def test_k4_of_screened_plans_uses_kept_pairs():
    w = make_config(3, scale={"natoms": 6})
    sh = w.shells
    rng = np.random.default_rng(4)
    ns = len(sh.l)
    rows = rng.integers(0, ns, (500, 4))
    got = bench._k4(w, rows)
    kab = oplan.prim_pairs_kept(sh.centers, sh.prim_off, sh.exps, rows[:, 0], rows[:, 1])
    kcd = oplan.prim_pairs_kept(sh.centers, sh.prim_off, sh.exps, rows[:, 2], rows[:, 3])
    np.testing.assert_array_equal(got, kab * kcd)
    K = np.asarray(sh.nprim)
    full = K[rows[:, 0]] * K[rows[:, 1]] * K[rows[:, 2]] * K[rows[:, 3]]
    assert np.all(got <= full) and np.any(got < full)


def test_k4_of_explicit_lists_is_the_full_product():
    w = make_config(2, scale={"nquartets": 50})
    q = np.asarray(w.quartets)
    K = np.asarray(w.shells.nprim)
    np.testing.assert_array_equal(bench._k4(w, q), K[q[:, 0]] * K[q[:, 1]] * K[q[:, 2]] * K[q[:, 3]])
