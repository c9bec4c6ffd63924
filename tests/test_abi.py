"""The C-ABI library loads and exports every function include/eri.h declares (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "electron_repulsion_integrals_amd", "liberi_mi355x.so")


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "eri.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(eri_[A-Za-z_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("eri_build_quartets", "eri_compute_batch", "eri_digest_J", "eri_strerror", "eri_plan_destroy"):
        assert n in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(lib, n), n


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_strerror_and_argument_validation_without_gpu():
    from electron_repulsion_integrals_amd import _lib
    L = _lib.load()
    assert L.eri_strerror(0) == b"ok"
    assert b"invalid" in L.eri_strerror(-1)
    # a NULL plan pointer is rejected before any device call
    sz = ctypes.c_size_t(0)
    assert L.eri_build_quartets(None, 0, None, 0, 0.0, None, ctypes.byref(sz), None, None) == -1
    assert L.eri_compute_batch(None, 0, 0, None, 0, None) == -1
    assert L.eri_digest_J(None, None, 0, None, 0, None, ctypes.byref(sz), None) == -1
    assert L.eri_compute_range(None, 0, 0, 1, None, 0, None) == -1
    assert L.eri_plan_quartets(None, 0, 1, None, None) == -1
    assert L.eri_digest_JK(None, None, 0, None, 0, None, 0, None, ctypes.byref(sz), None) == -1
    assert L.eri_digest_J_range(None, 0, 0, 1, None, 0, None, 0, None, ctypes.byref(sz), None) == -1
    assert L.eri_compute_deriv(None, 0, 1, None, 0, None, ctypes.byref(sz), None) == -1
    assert L.eri_plan_set_streams(None, None, 0) == -1
    assert L.eri_fp64_fma_tflops(None, None) == -1
    assert L.eri_plan_destroy(None) == 0
    assert b"workspace" in L.eri_strerror(-6)


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_invalid_shells_rejected_on_host():
    """l > 4, K = 0, non-positive exponents and out-of-range quartet indices fail before any launch."""
    import numpy as np
    from electron_repulsion_integrals_amd import _lib
    from workloads.configs import _pack

    def try_build(sh, q=None, tau=0.0, flags=0):
        c = np.ascontiguousarray(sh.centers)
        l = np.ascontiguousarray(sh.l, dtype=np.int32)
        k = np.ascontiguousarray(sh.nprim, dtype=np.int32)
        o = np.ascontiguousarray(sh.prim_off, dtype=np.int32)
        e = np.ascontiguousarray(sh.exps)
        cf = np.ascontiguousarray(sh.coefs)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        s = _lib._Shells(len(l), c.ctypes.data_as(dp), l.ctypes.data_as(ip), k.ctypes.data_as(ip),
                         o.ctypes.data_as(ip), e.ctypes.data_as(dp), cf.ctypes.data_as(dp))
        qq = None
        nq = 0
        if q is not None:
            qa = np.ascontiguousarray(np.asarray(q, dtype=np.int32).reshape(-1, 4))
            qq = qa.ctypes.data_as(ip)
            nq = len(qa)
        sz = ctypes.c_size_t(0)
        return _lib.load().eri_build_quartets(ctypes.byref(s), flags, qq, nq, tau, None, ctypes.byref(sz), None, None)

    good = dict(centers=[[0, 0, 0]], ls=[1], ks=[1], ex=[np.array([1.0])], co=[np.array([1.0])])
    assert try_build(_pack([[0, 0, 0]], [5], [1], [np.array([1.0])], [np.array([1.0])])) == -1
    assert try_build(_pack([[0, 0, 0]], [1], [1], [np.array([-1.0])], [np.array([1.0])])) == -1
    assert try_build(_pack([[0, 0, 0]], [1], [1], [np.array([1.0])], [np.array([1.0])]), q=[0, 0, 0, 1]) == -1
    assert try_build(_pack([[0, 0, np.nan]], [1], [1], [np.array([1.0])], [np.array([1.0])])) == -1
    assert try_build(_pack([[0, 0, 0]], [1], [1], [np.array([1.0])], [np.array([1.0])]), tau=-1.0) == -1
    # unknown flag bits fail; a screen with an explicit list fails
    one = _pack([[0, 0, 0]], [1], [1], [np.array([1.0])], [np.array([1.0])])
    assert try_build(one, flags=4) == -1
    assert try_build(one, flags=64) == -1
    assert try_build(one, q=[0, 0, 0, 0], tau=1e-12) == -1
    del good


@pytest.mark.gpu
def test_workspace_size_queries():
    """With a NULL workspace eri_build_quartets only adds up bytes on the host
    (hipCUB's temp-size queries read the device's properties, so a device must
    be visible): it writes no plan, grows with the quartet count, and a
    screened plan's size does not depend on tau (its slot lists are counts)."""
    import numpy as np
    from electron_repulsion_integrals_amd import _lib
    from workloads import make_config

    def query(w, q=None, tau=0.0, flags=0):
        sh = w.shells
        c = np.ascontiguousarray(sh.centers)
        l = np.ascontiguousarray(sh.l, dtype=np.int32)
        k = np.ascontiguousarray(sh.nprim, dtype=np.int32)
        o = np.ascontiguousarray(sh.prim_off, dtype=np.int32)
        e = np.ascontiguousarray(sh.exps)
        cf = np.ascontiguousarray(sh.coefs)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        s = _lib._Shells(len(l), c.ctypes.data_as(dp), l.ctypes.data_as(ip), k.ctypes.data_as(ip),
                         o.ctypes.data_as(ip), e.ctypes.data_as(dp), cf.ctypes.data_as(dp))
        qq, nq = None, 0
        if q is not None:
            qa = np.ascontiguousarray(np.asarray(q, dtype=np.int32).reshape(-1, 4))
            qq, nq = qa.ctypes.data_as(ip), len(qa)
        sz = ctypes.c_size_t(0)
        h = ctypes.c_void_p(1234)
        rc = _lib.load().eri_build_quartets(ctypes.byref(s), flags, qq, nq, tau, None, ctypes.byref(sz), None,
                                            ctypes.byref(h))
        assert rc == 0 and h.value == 1234
        return sz.value

    w2 = make_config(2, scale={"nquartets": 100})
    a, b = query(w2, w2.quartets[:50], flags=1), query(w2, w2.quartets, flags=1)
    assert 0 < a < b
    w3 = make_config(3, scale={"natoms": 4})
    assert query(w3, tau=1e-12, flags=1) == query(w3, tau=1e-3, flags=1) > 0
