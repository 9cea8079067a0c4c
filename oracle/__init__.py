"""Plain fp64 CPU oracle for the row-wise log-softmax heads (test infrastructure).

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does: it shares
no code with the HIP path.  The arithmetic lives in ``oracle.c`` (textbook
two-pass definitions in double precision); this module only marshals numpy
arrays through ctypes.

Every function takes the exact fp64 values of the stored logits (a bf16 or
fp32 tensor converted with ``.double()`` is exact) and returns fp64 results.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, invariants, brute force on tiny rows, finite differences
and independent library routines (torch fp64 ``log_softmax``, ``kl_div``,
autograd).  The gradient on a reverse-KL support-mismatch row (NaN on the
policy's support, 0 off it) is pinned by the limit of finite rows, up to the
NaN marker; its one corner without a pin (the reference masks all of the
policy's support, where the finite gradients converge) is marked "parity
unpinned" there.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

KL_REVERSE = 0
KL_FORWARD = 1

_lib = None


def build(out_path: str = LIB_PATH, extra_flags=()) -> str:
    """Compile oracle.c with gcc (no fast-math) into a shared library."""
    import subprocess

    src = os.path.join(_HERE, "oracle.c")
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           src, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def _load(path: str = LIB_PATH):
    lib = ctypes.CDLL(path)
    d = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    dbl = ctypes.c_double
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = None
    lib.orc_get_threads.argtypes = []
    lib.orc_get_threads.restype = ctypes.c_int
    lib.orc_softcap_fwd.argtypes = [d, i64, dbl, d]
    lib.orc_softcap_fwd.restype = None
    lib.orc_softcap_bwd.argtypes = [d, d, i64, dbl, d]
    lib.orc_softcap_bwd.restype = None
    lib.orc_logp_fwd.argtypes = [d, i64, i64, i64p, i64, dbl, d]
    lib.orc_logp_fwd.restype = ctypes.c_int
    lib.orc_logp_bwd.argtypes = [d, i64, i64, i64p, i64, dbl, d, d]
    lib.orc_logp_bwd.restype = ctypes.c_int
    lib.orc_entropy_fwd.argtypes = [d, i64, i64, dbl, d]
    lib.orc_entropy_fwd.restype = ctypes.c_int
    lib.orc_entropy_bwd.argtypes = [d, i64, i64, dbl, d, d]
    lib.orc_entropy_bwd.restype = ctypes.c_int
    lib.orc_kl_fwd.argtypes = [d, d, i64, i64, ctypes.c_int, dbl, dbl, d]
    lib.orc_kl_fwd.restype = ctypes.c_int
    lib.orc_kl_bwd.argtypes = [d, d, i64, i64, ctypes.c_int, dbl, dbl, d, d]
    lib.orc_kl_bwd.restype = ctypes.c_int
    lib.orc_kl_bwd_ref.argtypes = [d, d, i64, i64, ctypes.c_int, dbl, dbl, d, d]
    lib.orc_kl_bwd_ref.restype = ctypes.c_int
    return lib


class Oracle:
    """ctypes view of one compiled oracle library (the default or a variant)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: run __graft_entry__.build() (or oracle.build())")
        self.lib = _load(path)

    # -- helpers -------------------------------------------------------------
    @staticmethod
    def _d(a):
        a = np.ascontiguousarray(a, dtype=np.float64)
        return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))

    @staticmethod
    def _i(a):
        a = np.ascontiguousarray(a, dtype=np.int64)
        return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))

    @staticmethod
    def _check(rc):
        if rc != 0:
            raise MemoryError("oracle could not allocate its per-row buffers")

    def set_threads(self, n: int) -> None:
        self.lib.orc_set_threads(int(n))

    def threads(self) -> int:
        return int(self.lib.orc_get_threads())

    # -- softcap -------------------------------------------------------------
    def softcap_fwd(self, x, cap):
        x, px = self._d(x)
        y = np.empty_like(x)
        self.lib.orc_softcap_fwd(px, x.size, float(cap), self._d(y)[1])
        return y

    def softcap_bwd(self, x, grad_y, cap):
        x, px = self._d(x)
        gy, pg = self._d(grad_y)
        assert gy.shape == x.shape
        gx = np.empty_like(x)
        self.lib.orc_softcap_bwd(px, pg, x.size, float(cap), self._d(gx)[1])
        return gx

    # -- logprobs ------------------------------------------------------------
    def logp_fwd(self, x, targets, cap=0.0):
        """x [N, V]; targets [N] or [N, k] int64 -> logp of the same shape."""
        x, px = self._d(x)
        N, V = x.shape
        t = np.asarray(targets, dtype=np.int64)
        shape = t.shape
        t, pt = self._i(t.reshape(N, -1))
        k = t.shape[1]
        out = np.empty((N, k), dtype=np.float64)
        self._check(self.lib.orc_logp_fwd(px, N, V, pt, k, float(cap), self._d(out)[1]))
        return out.reshape(shape)

    def logp_bwd(self, x, targets, grad_out, cap=0.0):
        x, px = self._d(x)
        N, V = x.shape
        t, pt = self._i(np.asarray(targets, dtype=np.int64).reshape(N, -1))
        k = t.shape[1]
        g, pg = self._d(np.asarray(grad_out, dtype=np.float64).reshape(N, k))
        gx = np.empty((N, V), dtype=np.float64)
        self._check(self.lib.orc_logp_bwd(px, N, V, pt, k, float(cap), pg, self._d(gx)[1]))
        return gx

    # -- entropy -------------------------------------------------------------
    def entropy_fwd(self, x, cap=0.0):
        x, px = self._d(x)
        N, V = x.shape
        out = np.empty(N, dtype=np.float64)
        self._check(self.lib.orc_entropy_fwd(px, N, V, float(cap), self._d(out)[1]))
        return out

    def entropy_bwd(self, x, grad_out, cap=0.0):
        x, px = self._d(x)
        N, V = x.shape
        g, pg = self._d(np.asarray(grad_out, dtype=np.float64).reshape(N))
        gx = np.empty((N, V), dtype=np.float64)
        self._check(self.lib.orc_entropy_bwd(px, N, V, float(cap), pg, self._d(gx)[1]))
        return gx

    # -- KL ------------------------------------------------------------------
    def kl_fwd(self, pol, ref, direction=KL_REVERSE, cap_pol=0.0, cap_ref=0.0):
        pol, pp = self._d(pol)
        ref, pr = self._d(ref)
        assert pol.shape == ref.shape
        N, V = pol.shape
        out = np.empty(N, dtype=np.float64)
        self._check(self.lib.orc_kl_fwd(pp, pr, N, V, int(direction), float(cap_pol),
                                        float(cap_ref), self._d(out)[1]))
        return out

    def kl_bwd(self, pol, ref, grad_out, direction=KL_REVERSE, cap_pol=0.0, cap_ref=0.0):
        pol, pp = self._d(pol)
        ref, pr = self._d(ref)
        N, V = pol.shape
        g, pg = self._d(np.asarray(grad_out, dtype=np.float64).reshape(N))
        gx = np.empty((N, V), dtype=np.float64)
        self._check(self.lib.orc_kl_bwd(pp, pr, N, V, int(direction), float(cap_pol),
                                        float(cap_ref), pg, self._d(gx)[1]))
        return gx

    def kl_bwd_ref(self, pol, ref, grad_out, direction=KL_REVERSE, cap_pol=0.0, cap_ref=0.0):
        """Gradient of the KL with respect to the reference logits."""
        pol, pp = self._d(pol)
        ref, pr = self._d(ref)
        N, V = pol.shape
        g, pg = self._d(np.asarray(grad_out, dtype=np.float64).reshape(N))
        gr = np.empty((N, V), dtype=np.float64)
        self._check(self.lib.orc_kl_bwd_ref(pp, pr, N, V, int(direction), float(cap_pol),
                                            float(cap_ref), pg, self._d(gr)[1]))
        return gr


_default = None


def get() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default
