"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Bar (fp64): |gpu - oracle| <= max(1e-10 |oracle|, 1e-13) element by element;
plans (index maps) bit-exact against the oracle's plan twin fed the GPU's
Schwarz factors; Schwarz factors themselves to the same 1e-10 bar.
"""
import sys

import numpy as np
import pytest

import oracle
from oracle import plan as oplan
from workloads import make_config
from workloads.configs import _pack, subset_shells

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-10, 1e-13


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def eri():
    import torch
    assert torch.cuda.is_available()
    import electron_repulsion_integrals_amd as E
    E.load()
    return E


def assert_parity(got, ref, what=""):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = np.maximum(RTOL * np.abs(ref), ATOL)
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err / bound))
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} elements outside tolerance; worst at {i}: "
                             f"gpu={got.flat[i]!r} oracle={ref.flat[i]!r} err={err.flat[i]:.3e}")


def run_plan(E, sh, flags, quartets=None, tau=0.0):
    import torch
    plan = E.build_quartets(sh, flags, quartets, tau)
    out = torch.empty(max(plan.n_out, 1), dtype=torch.float64, device="cuda")
    E.compute_batch(plan, out)
    torch.cuda.synchronize()
    imap = plan.index_map().cpu().numpy() if plan.n_quartets else np.zeros((0, 5), np.int32)
    return plan, out[: plan.n_out].cpu().numpy(), imap


def oracle_flat(sh, imap, spherical):
    if len(imap) == 0:
        return np.zeros(0)
    flat, _ = oracle.eri(sh, imap[:, :4], spherical)
    return flat


def test_c1_all_unique_cartesian(eri):
    _log("case: C1 all unique quartets, Cartesian, screened mode tau=0")
    w = make_config(1)
    sh = w.shells
    plan, got, imap = run_plan(eri, sh, 0)
    assert plan.n_quartets == 666
    S_gpu = plan.schwarz().cpu().numpy()
    assert_parity(S_gpu, oracle.schwarz(sh, False), "Schwarz factors")
    twin = oplan.screened_plan(sh.l, sh.nprim, S_gpu, 0.0)
    np.testing.assert_array_equal(imap, twin["index_map"])
    assert [b[0] for b in twin["blocks"]] == list(plan.block_class)
    assert_parity(got, oracle_flat(sh, imap, False), "C1 integrals")


def _mixed_batch(seed, nshell, nq, lmax, kmax):
    rng = np.random.default_rng(seed)
    cen = rng.uniform(0, 6, (nshell, 3))
    ls = rng.integers(0, lmax + 1, nshell)
    ks = rng.integers(1, kmax + 1, nshell)
    ex = [np.exp(rng.uniform(np.log(0.1), np.log(30.0), k)) for k in ks]
    co = [rng.uniform(0.1, 1.0, k) for k in ks]
    sh = _pack(cen, ls, ks, ex, co)
    q = rng.integers(0, nshell, (nq, 4)).astype(np.int32)
    return sh, q


@pytest.mark.parametrize("spherical", [False, True])
def test_explicit_mixed_classes_l2(eri, spherical):
    _log(f"case: explicit mixed l<=2 batch, spherical={spherical}")
    sh, q = _mixed_batch(5, 30, 700, 2, 3)
    plan, got, imap = run_plan(eri, sh, 1 if spherical else 0, q)
    twin = oplan.explicit_plan(sh.l, sh.nprim, q)
    np.testing.assert_array_equal(imap, twin["index_map"])
    assert len(set(plan.block_class)) == 21
    assert_parity(got, oracle_flat(sh, imap, spherical), "mixed integrals")


def test_c2_dddd_reduced_full_compare(eri):
    _log("case: (dd|dd) x 333 spherical, full compare")
    w = make_config(2, scale={"nquartets": 333})
    plan, got, imap = run_plan(eri, w.shells, 1, w.quartets)
    assert plan.n_quartets == 333 and plan.n_blocks == 1
    assert_parity(got, oracle_flat(w.shells, imap, True), "dddd integrals")


def test_c2_full_size_sampled(eri):
    """20,000 (dd|dd) quartets in the benchmark's launch; oracle on a seeded sample."""
    _log("case: (dd|dd) x 20000 spherical, sampled compare")
    w = make_config(2)
    plan, got, imap = run_plan(eri, w.shells, 1, w.quartets)
    assert plan.n_quartets == 20000
    rng = np.random.default_rng(2)
    idx = np.unique(np.concatenate([[0, 1, 19998, 19999], rng.choice(20000, 300, replace=False)]))
    ref = oracle_flat(w.shells, imap[idx], True).reshape(len(idx), 625)
    assert_parity(got.reshape(20000, 625)[idx], ref, "dddd sampled")
    assert np.isfinite(got).all()


def test_single_quartet_and_long_contractions(eri):
    _log("case: single quartet with K=15 shells")
    rng = np.random.default_rng(9)
    ks = [15, 1, 15, 2]
    sh = _pack(rng.uniform(0, 3, (4, 3)), [2, 1, 2, 0], ks,
               [np.exp(rng.uniform(-2, 4, k)) for k in ks], [rng.uniform(0.1, 1, k) for k in ks])
    for spherical in (False, True):
        plan, got, imap = run_plan(eri, sh, 1 if spherical else 0, [[0, 1, 2, 3]])
        assert plan.n_quartets == 1
        assert_parity(got, oracle_flat(sh, imap, spherical), "single quartet")


def test_unnormalised_flag(eri):
    _log("case: ERI_NO_NORMALIZE")
    sh, q = _mixed_batch(11, 12, 120, 2, 2)
    plan, got, imap = run_plan(eri, sh, 2, q)
    ref, _ = oracle.eri(sh, imap[:, :4], False, normalize_=False)
    assert_parity(got, ref, "raw primitives")


def test_c3_reduced_plan_and_J(eri):
    """Screened plan + J digestion on a 4-atom cut of the SVP-like cluster."""
    import torch
    _log("case: C3 4-atom cluster, tau=1e-12, spherical, plan + J")
    w = make_config(3, scale={"natoms": 4})
    sh = w.shells
    plan, got, imap = run_plan(eri, sh, 1, None, w.tau)
    S_gpu = plan.schwarz().cpu().numpy()
    assert_parity(S_gpu, oracle.schwarz(sh, True), "Schwarz factors")
    twin = oplan.screened_plan(sh.l, sh.nprim, S_gpu, w.tau)
    np.testing.assert_array_equal(imap, twin["index_map"])
    flat = oracle_flat(sh, imap, True)
    assert_parity(got, flat, "C3 integrals")
    D = torch.tensor(w.density, device="cuda")
    J = torch.empty_like(D)
    eri.digest_J(plan, D, J)
    J2 = torch.empty_like(D)
    eri.digest_J(plan, D, J2)
    torch.cuda.synchronize()
    Jg = J.cpu().numpy()
    assert np.array_equal(Jg, J2.cpu().numpy()), "J is not bitwise reproducible"
    _, off = oracle.eri(sh, imap[:, :4], True)
    Jref = oracle.J_from_quartets(sh, True, imap[:, :4], flat, off, w.density)
    assert_parity(Jg, Jref, "J")
