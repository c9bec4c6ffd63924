"""The allocation-free J digestion (eri_digest_J_noalloc) against eri_digest_J.

eri_digest_J_noalloc keeps its chunk buffers in a file-scope device array
instead of a workspace, for callers that cannot allocate.  Called through the
C ABI twice in a row on one GPU -- the 4-atom SVP-like cluster, then the
smaller 2-atom cluster -- its J must equal eri_digest_J's J of the same plan to
the parity bar, be bitwise reproducible on a repeated call, and be symmetric to
the bar (within a diagonal shell block the two orientations come from
different horizontal-recurrence paths, so not bitwise).
"""
import ctypes

import numpy as np
import pytest

from workloads import make_config
from test_gpu_parity import assert_parity

pytestmark = pytest.mark.gpu


def _noalloc_J(E, plan, D):
    import torch
    L = E.load()
    L.eri_digest_J_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_int32, ctypes.c_void_p]
    L.eri_digest_J_noalloc.restype = ctypes.c_int
    J = torch.full_like(D, 7.0)  # every element is overwritten
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.eri_digest_J_noalloc(plan.handle, ctypes.c_void_p(D.data_ptr()), int(D.stride(0)),
                                ctypes.c_void_p(J.data_ptr()), int(J.stride(0)), stream)
    assert rc == 0, E.strerror(rc)
    return J


def test_noalloc_J_matches_digest_J_two_calls():
    import torch
    import electron_repulsion_integrals_amd as E
    E.load()
    for natoms in (4, 2):  # the second call has the smaller input
        print(f"case: noalloc J, {natoms}-atom SVP-like cluster", flush=True)
        w = make_config(3, scale={"natoms": natoms})
        plan = E.build_quartets(w.shells, E.ERI_SPHERICAL, None, w.tau)
        D = torch.tensor(w.density, device="cuda")
        Jref = torch.empty_like(D)
        E.digest_J(plan, D, Jref)
        J1 = _noalloc_J(E, plan, D)
        J2 = _noalloc_J(E, plan, D)
        torch.cuda.synchronize()
        a, b = J1.cpu().numpy(), J2.cpu().numpy()
        assert np.array_equal(a, b), "noalloc J is not bitwise reproducible"
        assert_parity(a, a.T, f"noalloc J symmetry, {natoms} atoms")
        assert_parity(a, Jref.cpu().numpy(), f"noalloc J vs eri_digest_J, {natoms} atoms")
