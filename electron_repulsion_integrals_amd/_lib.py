"""ctypes binding of liberi_mi355x.so (include/eri.h): argument marshalling only.

Every step of the integral path runs in the HIP library; this module converts
numpy shell arrays and torch device tensors into the C ABI's plain pointers
and raises on error codes.  The library allocates no device memory: the
workspaces its calls ask for (size queries with a NULL workspace) are torch
tensors allocated here and kept alive beside the plan.  There is no CPU
fallback: if the library is missing, loading fails with an error that says how
to build it.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liberi_mi355x.so")

ERI_SPHERICAL = 1
ERI_NO_NORMALIZE = 2
ERI_MAX_SIDE_STREAMS = 3
ERRORS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "capacity", -4: "HIP error", -5: "out of memory",
          -6: "workspace"}


class EriError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class _Shells(ctypes.Structure):
    _fields_ = [("nshell", ctypes.c_int32),
                ("centers", ctypes.POINTER(ctypes.c_double)),
                ("l", ctypes.POINTER(ctypes.c_int32)),
                ("nprim", ctypes.POINTER(ctypes.c_int32)),
                ("prim_off", ctypes.POINTER(ctypes.c_int32)),
                ("exps", ctypes.POINTER(ctypes.c_double)),
                ("coefs", ctypes.POINTER(ctypes.c_double))]


_lib = None
_lib_path = None


def load(path=None):
    """Load the library (once per process).  ``path`` selects another build of
    the same ABI, such as an ablation variant; a process holds one library."""
    global _lib, _lib_path
    if _lib is not None and path is None:
        return _lib
    path = os.path.abspath(path) if path else LIB_PATH
    if _lib is not None:
        if path != _lib_path:
            raise RuntimeError(f"{_lib_path} is already loaded in this process; cannot also load {path}")
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m electron_repulsion_integrals_amd.build`")
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    szp = ctypes.POINTER(ctypes.c_size_t)
    L.eri_build_quartets.argtypes = [ctypes.POINTER(_Shells), ctypes.c_int, i32p, ctypes.c_int64, ctypes.c_double,
                                     vp, szp, vp, ctypes.POINTER(vp)]
    L.eri_build_quartets.restype = ctypes.c_int
    L.eri_plan_set_streams.argtypes = [vp, ctypes.POINTER(vp), ctypes.c_int32]
    L.eri_plan_set_streams.restype = ctypes.c_int
    L.eri_plan_destroy.argtypes = [vp]
    L.eri_plan_destroy.restype = ctypes.c_int
    L.eri_plan_info.argtypes = [vp, i64p, i64p, i32p, i32p, i64p]
    L.eri_plan_info.restype = ctypes.c_int
    L.eri_plan_blocks.argtypes = [vp, i32p, i64p, i64p, i64p]
    L.eri_plan_blocks.restype = ctypes.c_int
    L.eri_plan_index_map.argtypes = [vp, vp, vp]
    L.eri_plan_index_map.restype = ctypes.c_int
    L.eri_plan_schwarz.argtypes = [vp, vp, vp]
    L.eri_plan_schwarz.restype = ctypes.c_int
    L.eri_compute_batch.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_int64, vp]
    L.eri_compute_batch.restype = ctypes.c_int
    L.eri_compute_range.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, vp, ctypes.c_int64, vp]
    L.eri_compute_range.restype = ctypes.c_int
    L.eri_plan_quartets.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, vp]
    L.eri_plan_quartets.restype = ctypes.c_int
    L.eri_digest_J.argtypes = [vp, vp, ctypes.c_int32, vp, ctypes.c_int32, vp, szp, vp]
    L.eri_digest_J.restype = ctypes.c_int
    L.eri_digest_J_range.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, vp, ctypes.c_int32, vp,
                                     ctypes.c_int32, vp, szp, vp]
    L.eri_digest_J_range.restype = ctypes.c_int
    L.eri_digest_JK.argtypes = [vp, vp, ctypes.c_int32, vp, ctypes.c_int32, vp, ctypes.c_int32, vp, szp, vp]
    L.eri_digest_JK.restype = ctypes.c_int
    L.eri_compute_deriv.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, ctypes.c_int64, vp, szp, vp]
    L.eri_compute_deriv.restype = ctypes.c_int
    L.eri_strerror.argtypes = [ctypes.c_int]
    L.eri_strerror.restype = ctypes.c_char_p
    L.eri_fp64_fma_tflops.argtypes = [ctypes.POINTER(ctypes.c_double), vp]
    L.eri_fp64_fma_tflops.restype = ctypes.c_int
    L.eri_class_info.argtypes = [ctypes.c_int32, i32p, i32p]
    L.eri_class_info.restype = ctypes.c_int
    _lib_path = path
    _lib = L
    return L


def _check(rc):
    if rc != 0:
        raise EriError(rc, load().eri_strerror(rc).decode())


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _workspace(nbytes):
    """A device workspace of at least nbytes (torch's allocator, 256-byte aligned)."""
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device="cuda")


class Plan:
    """A quartet plan: the library's host state plus the device workspace (a
    torch tensor held here) that holds its data; freed by close() or garbage
    collection."""

    def __init__(self, handle, workspace):
        self._h = handle
        self.workspace = workspace
        self._streams = []
        self._digest_ws = {}
        L = load()
        nq, nout, np_ = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        nb, nbf = ctypes.c_int32(), ctypes.c_int32()
        _check(L.eri_plan_info(self._h, ctypes.byref(nq), ctypes.byref(nout), ctypes.byref(nb), ctypes.byref(nbf),
                               ctypes.byref(np_)))
        self.n_quartets, self.n_out, self.n_blocks, self.nbf, self.n_pairs = \
            nq.value, nout.value, nb.value, nbf.value, np_.value
        n = self.n_blocks
        self.block_class = np.zeros(n, dtype=np.int32)
        self.block_start = np.zeros(n, dtype=np.int64)
        self.block_count = np.zeros(n, dtype=np.int64)
        self.block_out = np.zeros(n, dtype=np.int64)
        if n:
            _check(L.eri_plan_blocks(self._h, self.block_class.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     self.block_start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     self.block_count.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     self.block_out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan is closed")
        return self._h

    def close(self):
        if self._h is not None:
            load().eri_plan_destroy(self._h)
            self._h = None
        self.workspace = None
        self._digest_ws = {}

    def set_streams(self, streams):
        """Side streams (torch.cuda.Stream, at most ERI_MAX_SIDE_STREAMS) on which
        multi-block calls of this plan may run concurrently with the caller's stream."""
        streams = list(streams)
        arr = (ctypes.c_void_p * max(1, len(streams)))(*[s.cuda_stream for s in streams])
        _check(load().eri_plan_set_streams(self.handle, arr, len(streams)))
        self._streams = streams
        self._digest_ws = {}

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def index_map(self, stream=None):
        import torch
        out = torch.empty((self.n_quartets, 5), dtype=torch.int32, device="cuda")
        _check(load().eri_plan_index_map(self.handle, _ptr(out), _stream_handle(stream)))
        return out

    def quartets(self, first: int, count: int, stream=None):
        """Index-map rows of plan slots [first, first + count) as a (count, 5) int32 device tensor."""
        import torch
        out = torch.empty((int(count), 5), dtype=torch.int32, device="cuda")
        _check(load().eri_plan_quartets(self.handle, int(first), int(count), _ptr(out), _stream_handle(stream)))
        return out

    def schwarz(self, stream=None):
        import torch
        out = torch.empty(self.n_pairs, dtype=torch.float64, device="cuda")
        _check(load().eri_plan_schwarz(self.handle, _ptr(out), _stream_handle(stream)))
        return out


def build_quartets(shells, flags: int, quartets=None, tau: float = 0.0, stream=None,
                   side_streams: int = ERI_MAX_SIDE_STREAMS) -> Plan:
    """shells: object with centers, l, nprim, prim_off, exps, coefs (host arrays).

    The plan's workspace is a torch tensor sized by the library's query;
    ``side_streams`` new torch streams (default priority) are registered on the
    plan for its multi-block calls."""
    L = load()
    c = np.ascontiguousarray(shells.centers, dtype=np.float64)
    l = np.ascontiguousarray(shells.l, dtype=np.int32)
    k = np.ascontiguousarray(shells.nprim, dtype=np.int32)
    o = np.ascontiguousarray(shells.prim_off, dtype=np.int32)
    e = np.ascontiguousarray(shells.exps, dtype=np.float64)
    cf = np.ascontiguousarray(shells.coefs, dtype=np.float64)
    sh = _Shells(len(l), c.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                 l.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), k.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                 o.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), e.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                 cf.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    qptr = None
    nq = 0
    if quartets is not None:
        q = np.ascontiguousarray(np.asarray(quartets).reshape(-1, 4), dtype=np.int32)
        qptr = q.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        nq = len(q)
    h = ctypes.c_void_p()
    nbytes = ctypes.c_size_t(0)
    st = _stream_handle(stream)
    _check(L.eri_build_quartets(ctypes.byref(sh), int(flags), qptr, nq, float(tau), None, ctypes.byref(nbytes), st,
                                None))
    ws = _workspace(nbytes.value)
    nbytes = ctypes.c_size_t(ws.numel())
    _check(L.eri_build_quartets(ctypes.byref(sh), int(flags), qptr, nq, float(tau), _ptr(ws), ctypes.byref(nbytes),
                                st, ctypes.byref(h)))
    plan = Plan(h, ws)
    if side_streams:
        import torch
        plan.set_streams([torch.cuda.Stream() for _ in range(int(side_streams))])
    return plan


def compute_batch(plan: Plan, out, block_begin: int = 0, block_end: int | None = None, stream=None):
    """Integrals of blocks [block_begin, block_end) into the float64 device tensor ``out``."""
    if block_end is None:
        block_end = plan.n_blocks
    _check(load().eri_compute_batch(plan.handle, int(block_begin), int(block_end), _ptr(out), out.numel(),
                                    _stream_handle(stream)))
    return out


def compute_range(plan: Plan, block: int, first: int, count: int, out, stream=None):
    """Integrals of quartets [first, first + count) of one class block into ``out``."""
    _check(load().eri_compute_range(plan.handle, int(block), int(first), int(count), _ptr(out), out.numel(),
                                    _stream_handle(stream)))
    return out


def compute_deriv(plan: Plan, out, first: int = 0, count: int | None = None, stream=None):
    """First derivatives (12 blocks per slot: d/dA_x .. d/dD_z) of plan slots
    [first, first + count) into the float64 device tensor ``out``."""
    if count is None:
        count = plan.n_quartets - first
    L = load()
    st = _stream_handle(stream)
    nbytes = ctypes.c_size_t(0)
    _check(L.eri_compute_deriv(plan.handle, int(first), int(count), None, 0, None, ctypes.byref(nbytes), st))
    ws = _workspace(nbytes.value)
    nbytes = ctypes.c_size_t(ws.numel())
    _check(L.eri_compute_deriv(plan.handle, int(first), int(count), _ptr(out), out.numel(), _ptr(ws),
                               ctypes.byref(nbytes), st))
    return out


def _digest_workspace(plan: Plan, key, query):
    """The plan's digestion workspace for (J, K) wanted, sized by the library's
    query and kept for later calls of the same kind."""
    ws = plan._digest_ws.get(key)
    if ws is None:
        nbytes = ctypes.c_size_t(0)
        _check(query(ctypes.byref(nbytes)))
        ws = plan._digest_ws[key] = _workspace(nbytes.value)
    return ws


def digest_J(plan: Plan, D, J, stream=None):
    """J (device, nbf x nbf, float64) from the symmetric density D (device)."""
    L = load()
    st = _stream_handle(stream)
    ws = _digest_workspace(plan, (True, False), lambda nb: L.eri_digest_J(plan.handle, None, 0, None, 0, None, nb, st))
    nbytes = ctypes.c_size_t(ws.numel())
    _check(L.eri_digest_J(plan.handle, _ptr(D), int(D.stride(0)), _ptr(J), int(J.stride(0)), _ptr(ws),
                          ctypes.byref(nbytes), st))
    return J


def digest_J_range(plan: Plan, block: int, first: int, count: int, D, J, stream=None):
    """J (device, nbf x nbf, float64) += the Coulomb contributions of quartets
    [first, first + count) of class block ``block``; J is not cleared."""
    L = load()
    st = _stream_handle(stream)
    ws = _digest_workspace(plan, (True, False), lambda nb: L.eri_digest_J(plan.handle, None, 0, None, 0, None, nb, st))
    nbytes = ctypes.c_size_t(ws.numel())
    _check(L.eri_digest_J_range(plan.handle, int(block), int(first), int(count), _ptr(D), int(D.stride(0)), _ptr(J),
                                int(J.stride(0)), _ptr(ws), ctypes.byref(nbytes), st))
    return J


def digest_JK(plan: Plan, D, J=None, K=None, stream=None):
    """J and/or K (device, nbf x nbf, float64) from the symmetric density D in one pass."""
    L = load()
    st = _stream_handle(stream)
    jp = _ptr(J) if J is not None else None
    kp = _ptr(K) if K is not None else None
    ldj = int(J.stride(0)) if J is not None else 0
    ldk = int(K.stride(0)) if K is not None else 0
    ws = _digest_workspace(plan, (J is not None, K is not None),
                           lambda nb: L.eri_digest_JK(plan.handle, None, 0, jp, ldj, kp, ldk, None, nb, st))
    nbytes = ctypes.c_size_t(ws.numel())
    _check(L.eri_digest_JK(plan.handle, _ptr(D), int(D.stride(0)), jp, ldj, kp, ldk, _ptr(ws), ctypes.byref(nbytes),
                           st))
    return J, K


def class_info(class_id: int):
    l4 = (ctypes.c_int32 * 4)()
    tier = ctypes.c_int32()
    _check(load().eri_class_info(int(class_id), l4, ctypes.byref(tier)))
    return tuple(l4), chr(tier.value)


def strerror(code: int) -> str:
    return load().eri_strerror(int(code)).decode()


def fp64_fma_tflops(stream=None) -> float:
    """Measured FP64 FMA rate of the current device (TFLOP/s)."""
    v = ctypes.c_double(0.0)
    _check(load().eri_fp64_fma_tflops(ctypes.byref(v), _stream_handle(stream)))
    return v.value
