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


class _Sh:
    def __init__(self, centers, exps_per_shell):
        self.centers = np.asarray(centers, dtype=np.float64)
        self.exps = np.concatenate([np.asarray(e, dtype=np.float64) for e in exps_per_shell])
        self.prim_off = np.concatenate([[0], np.cumsum([len(e) for e in exps_per_shell])])


def test_prim_pairs_kept_hand_cases():
    """Kept counts worked out by hand: q = alpha beta / (alpha + beta) |AB|^2."""
    sh = _Sh([[0, 0, 0], [10, 0, 0], [100, 0, 0], [15, 2, 1], [15, 2, 1]],
             [[1.0, 10.0], [1.0, 100.0], [1.0], [2.0], [2.0000001]])
    # |AB|^2 = 100: q(1,1) = 50, q(1,100) = 99.0, q(10,1) = 90.9 kept; q(10,100) = 909 dropped
    # |AB|^2 = 1e4 with (1, 1): q = 5,000 for every pair -> none within, the first pair is kept
    # the same shell twice: |AB|^2 = 0, all K^2 pairs kept
    # |AB|^2 = 225 + 4 + 1 = 230 exactly and alpha = beta = 2: q = 230 exactly, kept;
    # a hair larger exponent puts q above 230
    got = op.prim_pairs_kept(sh.centers, sh.prim_off, sh.exps, [0, 2, 1, 3, 4], [1, 0, 1, 0, 0])
    np.testing.assert_array_equal(got, [3, 1, 4, 1, 1])
    s2 = _Sh([[0, 0, 0], [15, 2, 1]], [[2.0], [2.0]])
    assert op.prim_pairs_kept(s2.centers, s2.prim_off, s2.exps, [1], [0])[0] == 1
    s3 = _Sh([[0, 0, 0], [15, 2, 1]], [[2.0, 2.0000001], [2.0, 2.0000001]])
    # pairs (2, 2) -> q = 230 kept; any pair with 2.0000001 lies above
    assert op.prim_pairs_kept(s3.centers, s3.prim_off, s3.exps, [1], [0])[0] == 1
    s4 = _Sh([[0, 0, 0], [15, 2, 1]], [[2.0, 1.0], [2.0, 1.0]])
    # (2,2): 230 kept; (2,1) and (1,2): 2/3 * 230 kept; (1,1): 115 kept
    assert op.prim_pairs_kept(s4.centers, s4.prim_off, s4.exps, [1], [0])[0] == 4


def test_kept_counts_order_the_buckets():
    """With shells given, a pair's K is its kept count: two pairs of the same
    class and shell contraction degrees land in different buckets when one of
    them is far apart."""
    cen = [[0, 0, 0], [0, 0, 1], [0, 0, 50]]
    sh = _Sh(cen, [[1.0, 4.0], [1.0, 4.0], [1.0, 4.0]])
    l = np.zeros(3, dtype=int)
    K = np.full(3, 2)
    S = np.ones(6)
    pt_all = op.pair_table(l, K, S)
    pt = op.pair_table(l, K, S, shells=sh)
    assert set(pt_all["pairs"][:, 5]) == {4}
    kept = {(int(a), int(b)): int(k) for a, b, k in pt["pairs"][:, [2, 3, 5]]}
    # |AB|^2 = 1: every q <= 2; |AB|^2 = 2,500 or 2,401: q >= 1,200, none kept -> 1
    assert kept[(1, 0)] == 4 and kept[(0, 0)] == 4 and kept[(2, 2)] == 4
    assert kept[(2, 0)] == 1 and kept[(2, 1)] == 1
    full = op.screened_plan(l, K, S, 0.0, shells=sh)
    sc = op.screened_counts(l, K, S, 0.0, shells=sh)
    # one class block, ordered by (K_bra, K_ket): the far pairs (K = 1) lead
    kk = [(kept[tuple(sorted(r[:2], reverse=True))], kept[tuple(sorted(r[2:4], reverse=True))])
          for r in full["index_map"]]
    assert kk == sorted(kk) and kk[0] == (1, 1) and kk[-1] == (4, 4)
    np.testing.assert_array_equal(op.screened_decode(sc, np.arange(sc["n_quartets"])), full["index_map"])
