"""The oracle's counting form of the screened plan (for plans too large to
list) against its full enumeration: same quartet count, same class blocks,
and slot-by-slot the same index-map rows, including ties in S and products
that equal tau^2 exactly (kept, by the rule fl(S_p S_q) >= fl(tau^2))."""
import numpy as np
import pytest

from oracle import plan as op


def _case(seed):
    rng = np.random.default_rng(seed)
    ns = int(rng.integers(3, 14))
    l = rng.integers(0, 4, ns)
    K = rng.integers(1, 4, ns)
    npair = ns * (ns + 1) // 2
    S = rng.uniform(1e-8, 1.0, npair)
    S[rng.integers(0, npair, 4)] = S[1]  # ties inside buckets
    return l, K, S, float(rng.uniform(1e-6, 0.3))


@pytest.mark.parametrize("seed", range(8))
def test_counts_and_decode_match_enumeration(seed):
    l, K, S, tau = _case(seed)
    full = op.screened_plan(l, K, S, tau)
    sc = op.screened_counts(l, K, S, tau)
    assert sc["n_quartets"] == len(full["index_map"])
    assert [tuple(b) for b in sc["blocks"]] == [tuple(b) for b in full["blocks"]]
    rows = op.screened_decode(sc, np.arange(sc["n_quartets"]))
    np.testing.assert_array_equal(rows, full["index_map"])


def test_exact_threshold_products_are_kept():
    # powers of two: S_p S_q == tau^2 exactly for several pairs
    ns = 5
    l = np.zeros(ns, dtype=int)
    K = np.ones(ns, dtype=int)
    npair = ns * (ns + 1) // 2
    S = np.array([2.0 ** -(p % 5) for p in range(npair)])
    tau = 0.25
    full = op.screened_plan(l, K, S, tau)
    sc = op.screened_counts(l, K, S, tau)
    brute = sum(1 for p in range(npair) for q in range(p + 1) if S[p] * S[q] >= tau * tau)
    assert sc["n_quartets"] == len(full["index_map"]) == brute
    np.testing.assert_array_equal(op.screened_decode(sc, np.arange(brute)), full["index_map"])


def test_tau_zero_keeps_every_unique_quartet():
    ns = 6
    rng = np.random.default_rng(1)
    l, K = rng.integers(0, 3, ns), rng.integers(1, 3, ns)
    npair = ns * (ns + 1) // 2
    sc = op.screened_counts(l, K, rng.uniform(0, 1, npair), 0.0)
    assert sc["n_quartets"] == npair * (npair + 1) // 2
