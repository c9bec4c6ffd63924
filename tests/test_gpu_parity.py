"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Bar (fp64), element by element:
    |gpu - oracle| <= max(1e-10 |oracle|, 1e-13, 4 * B + C)
where B is the oracle's first-order fp64 error floor of the two-phase method:
rounding the contracted [e0|f0] intermediates to fp64, propagated through the
unrolled horizontal recurrence (oracle.hgp_rounding_bound), and C the rounding
of their contraction sums over K4 primitive quartets, sqrt(K4 - 1) eps
sum |term| propagated the same way (oracle.contraction_rounding_bound; zero
at K4 = 1).  The floor only matters for diffuse high-l quartets far apart,
where it exceeds 1e-10 of the result; it is computed only for quartets that
miss the first two terms.  The factor 4 and C are what the binary128
adjudication of tests/test_oracle_quad.py supports.  Every check records how many elements needed the floor, and the
largest |gpu - oracle| / B among them, in parity_floor_usage.jsonl (tests/floor_log.py).
Plans (index maps) are bit-exact against the oracle's plan twin fed the GPU's
Schwarz factors.
"""
import sys

import numpy as np
import pytest

import oracle
from oracle import plan as oplan
from workloads import make_config
from workloads.configs import _pack, subset_shells

from floor_log import FLOOR_FACTOR, record

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


HGP_FLOOR_FACTOR = FLOOR_FACTOR


def assert_parity(got, ref, what="", sh=None, quartets=None, spherical=None):
    """Element-wise bar; with (sh, quartets, spherical) the blocks of ``ref`` are the
    quartets' blocks in order and the two-phase fp64 floor may be applied."""
    got = np.asarray(got, dtype=float).ravel()
    ref = np.asarray(ref, dtype=float).ravel()
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    tol = np.maximum(RTOL * np.abs(ref), ATOL)
    bad = err > tol
    n_floor = 0
    worst_B = 0.0
    if bad.any() and sh is not None:
        q = np.asarray(quartets).reshape(-1, 4)
        sizes = oracle.block_sizes(sh, q, spherical)
        offs = np.concatenate([[0], np.cumsum(sizes)])
        qbad = np.unique(np.searchsorted(offs, np.nonzero(bad)[0], side="right") - 1)
        for x in qbad:
            # bar 4 B + C, written as 4 (B + C / 4)
            B = oracle.hgp_rounding_bound(sh, q[x:x + 1], spherical) + \
                oracle.contraction_rounding_bound(sh, q[x:x + 1], spherical) / HGP_FLOOR_FACTOR
            sl = slice(offs[x], offs[x + 1])
            newtol = np.maximum(tol[sl], HGP_FLOOR_FACTOR * B)
            m = err[sl] > tol[sl]
            n_floor += int(np.sum(m & (err[sl] <= newtol)))
            if m.any():
                worst_B = max(worst_B, float(np.max(err[sl][m] / np.maximum(B[m], 1e-300))))
            tol[sl] = newtol
        bad = err > tol
    record(what, got.size, n_floor + int(bad.sum()), worst_B)
    if n_floor:
        _log(f"  {what}: {n_floor} of {got.size} elements within the two-phase fp64 floor only "
             f"(largest err/B {worst_B:.2f})")
    if bad.any():
        i = int(np.argmax(err / tol))
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} elements outside tolerance; worst at {i}: "
                             f"gpu={got[i]!r} oracle={ref[i]!r} err={err[i]:.3e} tol={tol[i]:.3e}")


def run_plan(E, sh, flags, quartets=None, tau=0.0):
    import torch
    plan = E.build_quartets(sh, flags, quartets, tau)
    out = torch.empty(max(plan.n_out, 1), dtype=torch.float64, device="cuda")
    E.compute_batch(plan, out)
    torch.cuda.synchronize()
    imap = plan.index_map().cpu().numpy() if plan.n_quartets else np.zeros((0, 5), np.int32)
    return plan, out[: plan.n_out].cpu().numpy(), imap


def assert_schwarz(S_gpu, sh, spherical, what="Schwarz factors"):
    """S_p = max |(mu nu|mu nu)|: compared with the oracle's, the per-pair floor taken
    from the diagonal elements of the (ij|ij) block."""
    S_ref = oracle.schwarz(sh, spherical)
    err = np.abs(S_gpu - S_ref)
    tol = np.maximum(RTOL * np.abs(S_ref), ATOL)
    bad = np.nonzero(err > tol)[0]
    worst_B = 0.0
    for p in bad:
        i = int((np.sqrt(8 * p + 1) - 1) // 2)
        while i * (i + 1) // 2 > p:
            i -= 1
        while (i + 1) * (i + 2) // 2 <= p:
            i += 1
        j = p - i * (i + 1) // 2
        B = oracle.hgp_rounding_bound(sh, [[i, j, i, j]], spherical)
        n = int(round(np.sqrt(B.size)))
        Bd = float(np.max(np.diag(B.reshape(n, n))))
        worst_B = max(worst_B, float(err[p]) / max(Bd, 1e-300))
        tol[p] = max(tol[p], HGP_FLOOR_FACTOR * Bd)
    record(what, len(S_ref), len(bad), worst_B,
           floor_pairs=[int(p) for p in bad][:16])
    if len(bad):
        _log(f"  {what}: {len(bad)} of {len(S_ref)} factors checked against the two-phase fp64 floor "
             f"(pairs {[int(p) for p in bad][:16]}, largest err/B {worst_B:.2f})")
    worst = np.argmax(err / tol)
    assert np.all(err <= tol), f"{what}: worst pair {worst}: gpu={S_gpu[worst]!r} oracle={S_ref[worst]!r}"


def assert_J_parity(Jg, Jref, sh, spherical, D, S, tau, what):
    """J element-wise against the bar; an element that misses max(1e-10|ref|, 1e-13)
    may use the two-phase floor propagated into J (oracle.hgp_rounding_bound_J:
    the per-integral floor B of every quartet the element sums, times |D|), with
    the factor of the integral bar."""
    Jg = np.asarray(Jg, dtype=float)
    err = np.abs(Jg - Jref)
    tol = np.maximum(RTOL * np.abs(Jref), ATOL)
    bad = np.argwhere(err > tol)
    bf = oracle.basis_offsets(sh, spherical)
    shell_of = np.searchsorted(bf, np.arange(bf[-1]), side="right") - 1
    blocks = sorted({(int(shell_of[m]), int(shell_of[n])) for m, n in bad})
    worst = 0.0
    if blocks:
        floors = oracle.hgp_rounding_bound_J(sh, spherical, blocks, D, S, tau)
        for (i, j), F in zip(blocks, floors):
            sl = (slice(bf[i], bf[i + 1]), slice(bf[j], bf[j + 1]))
            e, t = err[sl], tol[sl]
            m = e > t
            if m.any():
                worst = max(worst, float(np.max(e[m] / np.maximum(F[m], 1e-300))))
            tol[sl] = np.maximum(t, HGP_FLOOR_FACTOR * F)
    nbad = int(np.sum(err > tol))
    record(what, Jg.size, len(bad), worst, floor_blocks=len(blocks))
    if len(bad):
        _log(f"  {what}: {len(bad)} of {Jg.size} elements within the propagated two-phase floor only, in "
             f"{len(blocks)} shell blocks (largest err/F {worst:.3f})")
    if nbad:
        k = int(np.argmax(err / tol))
        raise AssertionError(f"{what}: {nbad} elements outside the bar; worst flat index {k}: gpu={Jg.flat[k]!r} "
                             f"oracle={Jref.flat[k]!r} err={err.flat[k]:.3e} tol={tol.flat[k]:.3e}")


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
    assert_schwarz(S_gpu, sh, False)
    twin = oplan.screened_plan(sh.l, sh.nprim, S_gpu, 0.0, shells=sh)
    np.testing.assert_array_equal(imap, twin["index_map"])
    assert [b[0] for b in twin["blocks"]] == list(plan.block_class)
    assert_parity(got, oracle_flat(sh, imap, False), "C1 integrals", sh, imap[:, :4], False)


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
    assert_parity(got, oracle_flat(sh, imap, spherical), "mixed integrals", sh, imap[:, :4], spherical)


def test_c2_dddd_reduced_full_compare(eri):
    _log("case: (dd|dd) x 333 spherical, full compare")
    w = make_config(2, scale={"nquartets": 333})
    plan, got, imap = run_plan(eri, w.shells, 1, w.quartets)
    assert plan.n_quartets == 333 and plan.n_blocks == 1
    assert_parity(got, oracle_flat(w.shells, imap, True), "dddd integrals", w.shells, imap[:, :4], True)


def test_c2_full_size_sampled(eri):
    """20,000 (dd|dd) quartets in the benchmark's launch; oracle on a seeded sample."""
    _log("case: (dd|dd) x 20000 spherical, sampled compare")
    w = make_config(2)
    plan, got, imap = run_plan(eri, w.shells, 1, w.quartets)
    assert plan.n_quartets == 20000
    rng = np.random.default_rng(2)
    idx = np.unique(np.concatenate([[0, 1, 19998, 19999], rng.choice(20000, 300, replace=False)]))
    ref = oracle_flat(w.shells, imap[idx], True).reshape(len(idx), 625)
    assert_parity(got.reshape(20000, 625)[idx], ref, "dddd sampled", w.shells, imap[idx, :4], True)
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
        assert_parity(got, oracle_flat(sh, imap, spherical), "single quartet", sh, imap[:, :4], spherical)


def test_long_contractions_f_and_g_classes(eri):
    """f and g classes at contraction degree 5-8 (K4 of 300-2,700 primitive
    quartets), so the contracted kernels run their primitive-chunk loops many
    times: (ff|ff), (gf|dd), (gg|ps), (fd|dp), (dd|dd) and (gg|dd), two
    orientations each, both output kinds, against the oracle in full."""
    _log("case: f/g classes with K = 5-8, explicit list, both output kinds")
    rng = np.random.default_rng(31)
    ls = [3, 3, 4, 4, 2, 2, 1, 0, 4]
    ks = [6, 7, 6, 8, 8, 6, 7, 8, 5]
    sh = _pack(rng.uniform(0, 2.5, (len(ls), 3)), ls, ks,
               [np.exp(rng.uniform(np.log(0.1), np.log(50), k)) for k in ks], [rng.uniform(0.1, 1, k) for k in ks])
    q = [[0, 1, 0, 1], [1, 0, 0, 1], [2, 0, 4, 5], [3, 1, 5, 4], [3, 2, 6, 7], [2, 3, 7, 6],
         [0, 4, 5, 6], [1, 5, 4, 6], [4, 5, 4, 5], [5, 4, 5, 4], [8, 2, 4, 5], [2, 8, 5, 4]]
    for spherical in (True, False):
        plan, got, imap = run_plan(eri, sh, 1 if spherical else 0, q)
        assert plan.n_quartets == len(q)
        assert_parity(got, oracle_flat(sh, imap, spherical), "long contractions f/g", sh, imap[:, :4], spherical)


def test_screened_plan_with_dropped_primitive_pairs(eri):
    """Three atoms 3-4 bohr apart with s, p, d shells of contraction degree 4-6
    and exponents from 0.05 to 1e4: many primitive pairs of the shell pairs
    across atoms lie beyond the primitive-pair screen. Every unique quartet
    (tau = 0) is compared with the oracle, which sums every primitive pair, and
    so is J; the plan equals the twin built from the kept counts."""
    import torch
    _log("case: screened plan with dropped primitive pairs, tau=0, spherical, plan + J")
    rng = np.random.default_rng(32)
    atoms = np.array([[0, 0, 0], [3.0, 0.5, 0], [0.5, 4.0, 1.0]])
    ls, ks, cen = [], [], []
    for a in range(3):
        for l, k in ((0, 6), (1, 5), (2, 4)):
            ls.append(l)
            ks.append(k)
            cen.append(atoms[a])
    sh = _pack(np.array(cen), ls, ks, [np.exp(rng.uniform(np.log(0.05), np.log(1e4), k)) for k in ks],
               [rng.uniform(0.1, 1, k) for k in ks])
    ns = len(ls)
    i, j = np.tril_indices(ns)
    kept = oplan.prim_pairs_kept(sh.centers, sh.prim_off, sh.exps, i, j)
    full = np.asarray(ks)[i] * np.asarray(ks)[j]
    assert (kept < full).sum() >= 10 and (kept == full).sum() >= 10
    plan, got, imap = run_plan(eri, sh, 1, None, 0.0)
    S_gpu = plan.schwarz().cpu().numpy()
    assert_schwarz(S_gpu, sh, True)
    twin = oplan.screened_plan(sh.l, sh.nprim, S_gpu, 0.0, shells=sh)
    np.testing.assert_array_equal(imap, twin["index_map"])
    npair = ns * (ns + 1) // 2
    assert plan.n_quartets == npair * (npair + 1) // 2
    flat = oracle_flat(sh, imap, True)
    assert_parity(got, flat, "screened plan, dropped primitive pairs", sh, imap[:, :4], True)
    nb = int(oracle.basis_offsets(sh, True)[-1])
    C = rng.standard_normal((nb, nb // 2))
    Dn = C @ C.T
    D = torch.tensor(Dn, device="cuda")
    J = torch.empty_like(D)
    eri.digest_J(plan, D, J)
    torch.cuda.synchronize()
    _, off = oracle.eri(sh, imap[:, :4], True)
    Jref = oracle.J_from_quartets(sh, True, imap[:, :4], flat, off, Dn)
    assert_J_parity(J.cpu().numpy(), Jref, sh, True, Dn, S_gpu, 0.0, "J, dropped primitive pairs")


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
    assert_schwarz(S_gpu, sh, True)
    twin = oplan.screened_plan(sh.l, sh.nprim, S_gpu, w.tau, shells=sh)
    np.testing.assert_array_equal(imap, twin["index_map"])
    flat = oracle_flat(sh, imap, True)
    assert_parity(got, flat, "C3 integrals", sh, imap[:, :4], True)
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


def test_J_by_slot_ranges(eri):
    """eri_digest_J_range over ranges that partition every class block (the
    first block in three slot ranges, one of them empty), added into one zeroed
    J, gives the oracle's J of the 4-atom cluster; an empty range adds nothing;
    ranges outside the plan are rejected."""
    import torch
    _log("case: C3 4-atom cluster, J from slot ranges")
    w = make_config(3, scale={"natoms": 4})
    sh = w.shells
    plan = eri.build_quartets(sh, 1, None, w.tau)
    nb = plan.n_blocks
    cnt = [int(c) for c in plan.block_count]
    assert nb >= 3 and cnt[0] >= 2
    D = torch.tensor(w.density, device="cuda")
    J = torch.zeros_like(D)
    h = cnt[0] // 2
    ranges = [(0, 0, h), (0, h, 0), (0, h, cnt[0] - h)] + [(b, 0, cnt[b]) for b in range(1, nb)]
    for b, f, n in ranges:
        before = J.clone()
        eri.digest_J_range(plan, b, f, n, D, J)
        if n == 0:
            torch.cuda.synchronize()
            assert torch.equal(J, before), "an empty range changed J"
    for bad in ((nb, 0, 0), (0, 0, cnt[0] + 1), (0, cnt[0], 1), (-1, 0, 0)):
        with pytest.raises(eri.EriError):
            eri.digest_J_range(plan, *bad, D, J)
    torch.cuda.synchronize()
    imap = plan.index_map().cpu().numpy()
    flat, off = oracle.eri(sh, imap[:, :4], True)
    Jref = oracle.J_from_quartets(sh, True, imap[:, :4], flat, off, w.density)
    assert_parity(J.cpu().numpy(), Jref, "J by slot ranges")


def test_multi_block_call_matches_block_by_block(eri):
    """A call over all class blocks (blocks spread over the plan's side streams)
    gives bitwise the integrals of one call per block, on the caller's stream,
    and repeats bitwise; the first call on a fresh stream sees them complete."""
    import torch
    _log("case: multi-block compute_batch vs block by block, 4-atom cluster")
    w = make_config(3, scale={"natoms": 4})
    plan = eri.build_quartets(w.shells, 1, None, w.tau)
    assert plan.n_blocks > 4
    one = torch.empty(plan.n_out, dtype=torch.float64, device="cuda")
    for b in range(plan.n_blocks):
        eri.compute_batch(plan, one[int(plan.block_out[b]):], b, b + 1)
    s = torch.cuda.Stream()
    outs = []
    for _ in range(2):
        o = torch.full((plan.n_out,), float("nan"), dtype=torch.float64, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            eri.compute_batch(plan, o, stream=s)
            host = o.to("cpu", non_blocking=False)
        outs.append(host.numpy())
    torch.cuda.synchronize()
    ref = one.cpu().numpy()
    for got in outs:
        assert np.array_equal(got, ref), "multi-block integrals differ from the block-by-block ones"


def test_small_chunks_match_default_chunks(eri):
    """The same screened plan with its slot lists expanded in chunks of 1000
    quartets (instead of one chunk): identical index map and integrals, J to the
    bar and bitwise reproducible."""
    import os
    import torch
    _log("case: C3 4-atom cluster, 1000-quartet chunks vs one chunk")
    w = make_config(3, scale={"natoms": 4})
    sh = w.shells
    pe, oute, ime = run_plan(eri, sh, 1, None, w.tau)
    os.environ["ERI_CHUNK_QUARTETS"] = "1000"
    try:
        pi = eri.build_quartets(sh, eri.ERI_SPHERICAL, None, w.tau)
    finally:
        del os.environ["ERI_CHUNK_QUARTETS"]
    assert pi.n_quartets == pe.n_quartets > 5000
    np.testing.assert_array_equal(pi.block_count, pe.block_count)
    np.testing.assert_array_equal(pi.index_map().cpu().numpy(), ime)
    mid = pe.n_quartets // 2
    np.testing.assert_array_equal(pi.quartets(mid, 777).cpu().numpy(), ime[mid:mid + 777])
    outi = torch.empty(pi.n_out, dtype=torch.float64, device="cuda")
    eri.compute_batch(pi, outi)
    torch.cuda.synchronize()
    assert np.array_equal(outi.cpu().numpy(), oute), "1000-quartet chunks give other integrals than one chunk"
    D = torch.tensor(w.density, device="cuda")
    J1 = torch.full_like(D, 3.0)
    eri.digest_J(pi, D, J1)
    J2 = torch.empty_like(D)
    eri.digest_J(pi, D, J2)
    torch.cuda.synchronize()
    Jg = J1.cpu().numpy()
    assert np.array_equal(Jg, J2.cpu().numpy()), "J is not bitwise reproducible"
    flat, off = oracle.eri(sh, ime[:, :4], True)
    Jref = oracle.J_from_quartets(sh, True, ime[:, :4], flat, off, w.density)
    assert_parity(Jg, Jref, "J with 1000-quartet chunks")


def test_K_tiny_molecule_against_plain_sum(eri):
    """Exchange K of the 4-centre s/p molecule (all unique quartets, Cartesian)
    against the oracle's plain four-index sum; J from the same pass against its
    plain sum; both bitwise reproducible."""
    import torch
    _log("case: K and J of the tiny s/p molecule, screened plan with tau = 0")
    w = make_config(1)
    sh = w.shells
    N = sh.nbf(False)
    rng = np.random.default_rng(11)
    C = rng.standard_normal((N, N // 4))
    Dh = C @ C.T
    plan = eri.build_quartets(sh, 0, None, 0.0)
    D = torch.tensor(Dh, device="cuda")
    J, K = torch.empty_like(D), torch.full_like(D, 5.0)
    eri.digest_JK(plan, D, J, K)
    J2, K2 = torch.empty_like(D), torch.empty_like(D)
    eri.digest_JK(plan, D, J2, K2)
    torch.cuda.synchronize()
    assert torch.equal(K, K2) and torch.equal(J, J2), "J/K are not bitwise reproducible"
    assert_parity(K.cpu().numpy(), oracle.K_naive(sh, False, Dh), "K vs plain sum")
    assert_parity(J.cpu().numpy(), oracle.J_naive(sh, False, Dh), "J (JK pass) vs plain sum")


def test_K_cluster_default_and_small_chunks(eri):
    """K of the 4-atom SVP-like cluster (spherical, tau = 1e-12) with one chunk
    and with 1000-quartet chunks, against the oracle's unique-quartet K over the
    same quartets."""
    import os
    import torch
    _log("case: K of the C3 4-atom cluster, one chunk and 1000-quartet chunks")
    w = make_config(3, scale={"natoms": 4})
    sh = w.shells
    pe = eri.build_quartets(sh, eri.ERI_SPHERICAL, None, w.tau)
    os.environ["ERI_CHUNK_QUARTETS"] = "1000"
    try:
        pi = eri.build_quartets(sh, eri.ERI_SPHERICAL, None, w.tau)
    finally:
        del os.environ["ERI_CHUNK_QUARTETS"]
    imap = pe.index_map().cpu().numpy()
    D = torch.tensor(w.density, device="cuda")
    Ke, Ki = torch.empty_like(D), torch.empty_like(D)
    eri.digest_JK(pe, D, None, Ke)
    eri.digest_JK(pi, D, None, Ki)
    torch.cuda.synchronize()
    flat, off = oracle.eri(sh, imap[:, :4], True)
    Kref = oracle.K_from_quartets(sh, True, imap[:, :4], flat, off, w.density)
    assert_parity(Ke.cpu().numpy(), Kref, "K one chunk")
    assert_parity(Ki.cpu().numpy(), Kref, "K 1000-quartet chunks")
    Kg = Ke.cpu().numpy()
    assert np.array_equal(Kg, Kg.T)


def _cheap_slots(rows, nprim, limit):
    k4 = np.prod(nprim[rows[:, :4]], axis=1)
    return k4 <= limit


def test_c5_full_plan_counts_and_sampled_integrals(eri):
    """The 120-atom TZVP-like cluster at full size (2e10 screened quartets, an
    implicit plan): quartet count and class blocks equal the oracle's counting
    twin fed the GPU's Schwarz factors; sampled slots decode to the twin's
    quartets; sampled Schwarz factors and integrals meet the bar."""
    import torch
    _log("case: C5 120-atom cluster, full implicit plan, sampled checks")
    w = make_config(5)
    sh = w.shells
    plan = eri.build_quartets(sh, eri.ERI_SPHERICAL, None, w.tau)
    S = plan.schwarz().cpu().numpy()
    _log(f"  plan: {plan.n_quartets} quartets, {plan.n_blocks} blocks")
    sc = oplan.screened_counts(sh.l, sh.nprim, S, w.tau, shells=sh)
    assert plan.n_quartets == sc["n_quartets"]
    assert [(int(c), int(s), int(n)) for c, s, n in zip(plan.block_class, plan.block_start, plan.block_count)] == \
        [tuple(int(v) for v in b) for b in sc["blocks"]]
    rng = np.random.default_rng(5)
    nprim = np.asarray(sh.nprim)
    # Schwarz factors of sampled pairs with modest contraction, by their definition
    ns = len(sh.l)
    pi = rng.integers(0, ns, 400)
    pj = rng.integers(0, ns, 400)
    i, j = np.maximum(pi, pj), np.minimum(pi, pj)
    sel = nprim[i] * nprim[j] <= 16
    i, j = i[sel][:60], j[sel][:60]
    flat, off = oracle.eri(sh, np.stack([i, j, i, j], axis=1), True)
    ends = np.append(np.asarray(off)[:len(i)], len(flat))
    Sref = np.array([np.abs(flat[ends[x]:ends[x + 1]]).max() for x in range(len(i))])
    assert_parity(S[i * (i + 1) // 2 + j], Sref, "C5 sampled Schwarz factors")
    # per block: the first slot, seeded slots of modest cost, and the seeded slot
    # with the largest primitive-quartet count
    out_rows, out_vals, k4max = [], [], []
    for b in range(plan.n_blocks):
        st, cnt = int(plan.block_start[b]), int(plan.block_count[b])
        cand = np.unique(np.concatenate([[st], st + rng.integers(0, cnt, 64)]))
        rows_all = oplan.screened_decode(sc, cand)
        got_rows = np.concatenate([plan.quartets(int(s), 1).cpu().numpy() for s in cand[:8]])
        np.testing.assert_array_equal(got_rows, rows_all[:8])
        keep = list(np.flatnonzero(_cheap_slots(rows_all, nprim, 64))[:3])
        # and the candidate with the longest contraction (K4 up to 8^4 in this cluster)
        k4 = np.prod(nprim[rows_all[:, :4]], axis=1)
        keep.append(int(np.argmax(k4)))
        k4max.append(int(k4.max()))
        for x in dict.fromkeys(keep):
            s = int(cand[x])
            n = int(oracle.block_sizes(sh, rows_all[x:x + 1, :4], True)[0])
            o = torch.empty(n, dtype=torch.float64, device="cuda")
            eri.compute_range(plan, b, s - st, 1, o)
            out_vals.append(o.cpu().numpy())
            out_rows.append(rows_all[x])
    torch.cuda.synchronize()
    q = np.array(out_rows)[:, :4]
    flat, _ = oracle.eri(sh, q, True)
    _log(f"  {len(q)} sampled quartets over {plan.n_blocks} blocks, largest K4 per block: {k4max}")
    assert max(k4max) >= 1024
    assert_parity(np.concatenate(out_vals), flat, "C5 sampled integrals", sh, q, True)


def test_all_120_classes_explicit(eri):
    """Every class up to (gg|gg), both output kinds, random shells with K <= 2."""
    _log("case: explicit mixed batch over all 120 classes")
    sh, q = _mixed_batch(21, 60, 4000, 4, 2)
    for spherical in (True, False):
        plan, got, imap = run_plan(eri, sh, 1 if spherical else 0, q)
        twin = oplan.explicit_plan(sh.l, sh.nprim, q)
        np.testing.assert_array_equal(imap, twin["index_map"])
        assert len(set(plan.block_class)) == 120
        assert_parity(got, oracle_flat(sh, imap, spherical), f"all classes sph={spherical}", sh, imap[:, :4], spherical)


def test_all_120_classes_uncontracted(eri):
    """Every class with uncontracted shells only, so that every block runs the
    K4 = 1 kernels (among them the packed multi-quartet workgroups of the
    classes whose bra spans 35 lanes); block sizes are ragged against the
    quartets per workgroup."""
    _log("case: explicit uncontracted batch over all 120 classes")
    sh, q = _mixed_batch(27, 60, 2500, 4, 1)
    for spherical in (True, False):
        plan, got, imap = run_plan(eri, sh, 1 if spherical else 0, q)
        assert len(set(plan.block_class)) == 120
        assert_parity(got, oracle_flat(sh, imap, spherical), f"uncontracted classes sph={spherical}", sh,
                      imap[:, :4], spherical)


def test_c4_reduced_full_compare(eri):
    _log("case: (ff|ff) x 64 + (gg|gg) x 16, K=2, spherical, full compare")
    w = make_config(4, scale={"nquartets_f": 64, "nquartets_g": 16})
    plan, got, imap = run_plan(eri, w.shells, 1, w.quartets)
    assert list(plan.block_count) == [64, 16]
    assert_parity(got, oracle_flat(w.shells, imap, True), "ff/gg integrals", w.shells, imap[:, :4], True)


def test_c4_full_size_sampled(eri):
    _log("case: (ff|ff) x 4000 + (gg|gg) x 1000 spherical, sampled compare")
    w = make_config(4)
    plan, got, imap = run_plan(eri, w.shells, 1, w.quartets)
    assert list(plan.block_count) == [4000, 1000]
    rng = np.random.default_rng(4)
    fsel = np.unique(np.concatenate([[0, 3999], rng.choice(4000, 400, replace=False)]))
    gsel = np.unique(np.concatenate([[4000, 4999], 4000 + rng.choice(1000, 100, replace=False)]))
    ff = got[: 4000 * 2401].reshape(4000, 2401)
    gg = got[4000 * 2401:].reshape(1000, 6561)
    assert_parity(ff[fsel], oracle_flat(w.shells, imap[fsel], True), "ffff sampled", w.shells, imap[fsel, :4], True)
    assert_parity(gg[gsel - 4000], oracle_flat(w.shells, imap[gsel], True), "gggg sampled", w.shells, imap[gsel, :4], True)
    assert np.isfinite(got).all()


def test_c3_full_size_plan_and_sampled_J(eri):
    """30-atom SVP-like cluster, tau = 1e-12: bit-exact plan, sampled integrals, sampled J blocks."""
    import torch
    _log("case: C3 full 30-atom cluster, plan + J")
    w = make_config(3)
    sh = w.shells
    plan = eri.build_quartets(sh, 1, None, w.tau)
    S_gpu = plan.schwarz().cpu().numpy()
    rng = np.random.default_rng(3)
    pairs_all = [(i, j) for i in range(sh.nshell) for j in range(i + 1)]
    psel = rng.choice(len(pairs_all), 60, replace=False)
    assert_schwarz(S_gpu, sh, True)
    imap = plan.index_map().cpu().numpy()
    twin = oplan.screened_plan(sh.l, sh.nprim, S_gpu, w.tau, shells=sh)
    np.testing.assert_array_equal(imap, twin["index_map"])
    _log(f"  plan: {plan.n_quartets} quartets in {plan.n_blocks} class blocks")
    # unique quartets whose Schwarz product lies within 1e-9 (relative) of tau^2, where
    # the keep/drop decision would be sensitive to the last digits of S
    Ss = np.sort(S_gpu)
    t2 = w.tau * w.tau
    lo = np.searchsorted(Ss, t2 * (1 - 1e-9) / np.maximum(Ss, 1e-300), side="left")
    hi = np.searchsorted(Ss, t2 * (1 + 1e-9) / np.maximum(Ss, 1e-300), side="right")
    near = int(np.sum(np.maximum(hi - lo, 0)))
    _log(f"  ordered pair-pair products within 1e-9 of tau^2: {near}")
    out = torch.empty(plan.n_out, dtype=torch.float64, device="cuda")
    eri.compute_batch(plan, out)
    D = torch.tensor(w.density, device="cuda")
    J = torch.empty_like(D)
    eri.digest_J(plan, D, J)
    torch.cuda.synchronize()
    # sampled integrals: 1500 quartets spread over every class block
    sizes = oracle.block_sizes(sh, imap[:, :4], True)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    qs = np.unique(np.concatenate([plan.block_start, plan.block_start + plan.block_count - 1,
                                   rng.choice(plan.n_quartets, 1500, replace=False)]))
    got = out.cpu().numpy()
    ref, roff = oracle.eri(sh, imap[qs, :4], True)
    g = np.concatenate([got[offs[x]: offs[x + 1]] for x in qs])
    assert_parity(g, ref, "C3 sampled integrals", sh, imap[qs, :4], True)
    # sampled J blocks by the plain sum over all ket pairs
    Jg = J.cpu().numpy()
    bf = oracle.basis_offsets(sh, True)
    bras = [pairs_all[x] for x in psel[:6]]
    refs = oracle.J_blocks(sh, True, bras, w.density, S_gpu, w.tau)
    for (i, j), Jb in zip(bras, refs):
        assert_parity(Jg[bf[i]:bf[i + 1], bf[j]:bf[j + 1]], Jb, f"J block ({i},{j})")
        assert_parity(Jg[bf[j]:bf[j + 1], bf[i]:bf[i + 1]], Jb.T, f"J block ({j},{i})")


def test_c3_full_size_JK(eri):
    """30-atom SVP-like cluster, tau = 1e-12: J and K in one pass; J agrees with
    eri_digest_J's, sampled K blocks (diagonal and off-diagonal shell pairs)
    against the plain sum over every (j, l) shell pair, K symmetric."""
    import torch
    _log("case: C3 full 30-atom cluster, J and K in one pass")
    w = make_config(3)
    sh = w.shells
    plan = eri.build_quartets(sh, 1, None, w.tau)
    S_gpu = plan.schwarz().cpu().numpy()
    D = torch.tensor(w.density, device="cuda")
    J0, J, K = torch.empty_like(D), torch.empty_like(D), torch.empty_like(D)
    eri.digest_J(plan, D, J0)
    eri.digest_JK(plan, D, J, K)
    torch.cuda.synchronize()
    assert_parity(J.cpu().numpy(), J0.cpu().numpy(), "J of the JK pass vs eri_digest_J")
    Kg = K.cpu().numpy()
    assert np.array_equal(Kg, Kg.T)
    rng = np.random.default_rng(31)
    ns = sh.nshell
    pairs = [(int(i), int(i)) for i in rng.choice(ns, 2, replace=False)] + \
            [(int(i), int(k)) for i, k in zip(rng.choice(ns, 3, replace=False), rng.choice(ns, 3, replace=False))]
    bf = oracle.basis_offsets(sh, True)
    for (i, k), Kb in zip(pairs, oracle.K_blocks(sh, True, pairs, w.density, S_gpu, w.tau)):
        assert_parity(Kg[bf[i]:bf[i + 1], bf[k]:bf[k + 1]], Kb, f"K block ({i},{k})")


def test_c3_full_J_against_oracle_fixture(eri):
    """The full J of the 30-atom SVP-like cluster (10.2 M screened quartets)
    against the oracle's full J element by element; the oracle's J is stored in
    tests/golden/c3_J_spherical.npz by tests/golden/make_c3_J.py, which calls
    only the oracle (its own Schwarz factors, screened plan, four-index
    integrals and unique-quartet digestion).  The workspace of the plan and of
    the digestion are torch tensors the binding allocates from the library's
    size queries."""
    import os
    import torch
    _log("case: C3 full 30-atom cluster, full J against the oracle's full J")
    fx = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "c3_J_spherical.npz"))
    w = make_config(3)
    plan = eri.build_quartets(w.shells, eri.ERI_SPHERICAL, None, w.tau)
    assert plan.workspace.numel() > 0
    D = torch.tensor(w.density, device="cuda")
    J = torch.empty_like(D)
    eri.digest_J(plan, D, J)
    torch.cuda.synchronize()
    _log(f"  {plan.n_quartets} quartets (oracle plan: {int(fx['n_quartets'])})")
    assert abs(plan.n_quartets - int(fx["n_quartets"])) <= 10
    S = plan.schwarz().cpu().numpy()
    assert_J_parity(J.cpu().numpy(), fx["J"], w.shells, True, w.density, S, w.tau, "C3 full J vs oracle")


def test_c5_shape_cluster_J(eri):
    """J of an 8-atom cluster with the 120-atom cluster's per-atom shells (5s 4p
    3d 1f, K 1-8, exponents [0.05, 1e4], atoms in the same 35-bohr cube,
    tau = 1e-12, spherical) through eri_digest_J; 16 seeded bra shell
    pairs' J blocks (both orientations) against the oracle's plain sum over
    every surviving ket pair; sampled Schwarz factors against the oracle's."""
    import torch
    _log("case: C5-shape 8-atom cluster, J blocks of 16 seeded bra pairs")
    w = make_config(5, scale={"natoms": 8})
    sh = w.shells
    plan = eri.build_quartets(sh, eri.ERI_SPHERICAL, None, w.tau)
    S = plan.schwarz().cpu().numpy()
    D = torch.tensor(w.density, device="cuda")
    J = torch.empty_like(D)
    eri.digest_J(plan, D, J)
    torch.cuda.synchronize()
    _log(f"  {plan.n_quartets} quartets in {plan.n_blocks} class blocks")
    rng = np.random.default_rng(55)
    pairs = [(i, j) for i in range(sh.nshell) for j in range(i + 1)]
    bras = [pairs[x] for x in rng.choice(len(pairs), 16, replace=False)]
    nprim = np.asarray(sh.nprim)
    cheap = [p for p in pairs if nprim[p[0]] * nprim[p[1]] <= 16]
    sp = [cheap[x] for x in rng.choice(len(cheap), 24, replace=False)]
    flat, off = oracle.eri(sh, [(i, j, i, j) for i, j in sp], True)
    ends = np.append(np.asarray(off), len(flat))
    Sref = np.array([np.abs(np.diag(flat[ends[x]:ends[x + 1]].reshape(
        int(round(np.sqrt(ends[x + 1] - ends[x]))), -1))).max() for x in range(len(sp))])
    assert_parity(S[[i * (i + 1) // 2 + j for i, j in sp]], Sref, "C5-shape sampled Schwarz factors")
    Jg = J.cpu().numpy()
    bf = oracle.basis_offsets(sh, True)
    refs = oracle.J_blocks(sh, True, bras, w.density, S, w.tau)
    for (i, j), Jb in zip(bras, refs):
        assert_parity(Jg[bf[i]:bf[i + 1], bf[j]:bf[j + 1]], Jb, f"C5-shape J block ({i},{j})")
        assert_parity(Jg[bf[j]:bf[j + 1], bf[i]:bf[i + 1]], Jb.T, f"C5-shape J block ({j},{i})")
