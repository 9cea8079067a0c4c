"""The C ABI on the host (no GPU needed): exports, helpers and validation.

Every argument check of include/rlk.h runs on the host before any HIP call,
so the error codes and the empty-input path are testable without a GPU.
"""

import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

from vocab_log_softmax_amd import rlk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ARG, DTYPE, SHAPE, DEVICE = 0, 1, 2, 3, 4
F = ctypes.c_float


@pytest.fixture(scope="module")
def lib():
    return rlk.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "rlk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlk_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("rlk_softcap_fwd", "rlk_softcap_bwd", "rlk_logp_fwd", "rlk_logp_bwd",
               "rlk_entropy_fwd", "rlk_entropy_bwd", "rlk_kl_fwd", "rlk_kl_bwd"):
        assert fn in names
    assert set(names) == set(rlk.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for fn in declared_functions():
        assert hasattr(lib, fn), fn


def test_helpers(lib):
    assert lib.rlk_abi_version() == 1
    assert lib.rlk_stats_bytes(0, 10, 7) == 320
    assert lib.rlk_stats_bytes(2, 3, 7) == 96
    assert lib.rlk_stats_bytes(0, 0, 7) == 0
    assert lib.rlk_stats_bytes(9, 3, 7) == 0
    assert lib.rlk_status_str(3) == b"RLK_ERR_SHAPE"
    assert lib.rlk_status_str(42) == b"RLK_ERR_UNKNOWN"


def _logp_fwd(lib, dtype=1, N=4, V=10, ld=10, k=1, cap=0.0, ptrs=True):
    p = ctypes.c_void_p(16) if ptrs else None
    return lib.rlk_logp_fwd(p, dtype, N, V, ld, p, k, F(cap), p, p, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(N=-1), SHAPE), (dict(V=0), SHAPE), (dict(ld=9), SHAPE), (dict(V=2**31, ld=2**31), SHAPE),
    (dict(k=0), SHAPE), (dict(k=4097), SHAPE), (dict(N=2**40, ld=2**30, V=10), SHAPE),
    (dict(cap=-1.0), ARG), (dict(cap=float("nan")), ARG), (dict(cap=float("inf")), ARG),
    (dict(ptrs=False), ARG),
])
def test_logp_fwd_rejects(lib, kw, code):
    assert _logp_fwd(lib, **kw) == code
    assert rlk.rlk_last_error() != ""


def test_empty_inputs_launch_nothing(lib):
    # N == 0 is OK even with null pointers: nothing is touched, no HIP call.
    assert _logp_fwd(lib, N=0, ptrs=False) == OK
    assert lib.rlk_logp_bwd(None, 0, 0, 5, 5, None, 3, F(20.0), None, None, None, None) == OK
    assert lib.rlk_entropy_fwd(None, 1, 0, 5, 5, F(0), None, None, None) == OK
    assert lib.rlk_entropy_bwd(None, 1, 0, 5, 5, F(0), None, None, None, None) == OK
    assert lib.rlk_kl_fwd(None, None, 1, 0, 5, 5, 5, 0, F(0), F(0), None, None, None) == OK
    assert lib.rlk_kl_bwd(None, None, 1, 0, 5, 5, 5, 1, F(0), F(0), None, None, None, None) == OK
    assert lib.rlk_softcap_fwd(None, 1, None, 0, 0, F(30.0), None) == OK
    assert lib.rlk_softcap_bwd(None, 1, None, None, 0, F(30.0), None) == OK
    assert rlk.rlk_last_error() == ""


def test_other_entry_points_validate(lib):
    p = ctypes.c_void_p(16)
    assert lib.rlk_softcap_fwd(p, 1, p, 0, 8, F(0.0), None) == ARG        # cap must be > 0
    assert lib.rlk_softcap_fwd(p, 1, p, 3, 8, F(30.0), None) == DTYPE
    assert lib.rlk_softcap_fwd(p, 7, p, 0, 8, F(30.0), None) == DTYPE
    assert lib.rlk_softcap_bwd(p, 5, p, p, 8, F(30.0), None) == DTYPE
    assert lib.rlk_softcap_bwd(p, 1, p, p, -1, F(30.0), None) == SHAPE
    assert lib.rlk_entropy_fwd(p, 1, 4, 8, 7, F(0), p, p, None) == SHAPE   # ld < V
    assert lib.rlk_entropy_bwd(p, 1, 4, 8, 8, F(-3.0), p, p, p, None) == ARG
    assert lib.rlk_kl_fwd(p, p, 1, 4, 8, 8, 8, 2, F(0), F(0), p, p, None) == ARG  # bad dir
    assert lib.rlk_kl_fwd(p, p, 1, 4, 8, 8, 6, 0, F(0), F(0), p, p, None) == SHAPE
    assert lib.rlk_kl_bwd(p, p, 1, 4, 8, 8, 8, 0, F(0), F(float("nan")), p, p, p, None) == ARG
    assert lib.rlk_kl_bwd(p, p, 1, 4, 8, 8, 8, 0, F(0), F(0), p, None, p, None) == ARG


def test_host_memory_is_rejected_before_launch(lib):
    # Plain host memory is not device memory: RLK_ERR_DEVICE, nothing launched.
    x = np.zeros((4, 16), np.float32)
    t = np.zeros((4, 1), np.int64)
    o = np.zeros((4, 1), np.float32)
    s = np.zeros(128, np.uint8)
    st = lib.rlk_logp_fwd(x.ctypes.data, 0, 4, 16, 16, t.ctypes.data, 1, F(0), o.ctypes.data,
                          s.ctypes.data, None)
    assert st == DEVICE


def test_binding_raises_with_status():
    err = rlk.RLKError("rlk_logp_fwd", 3, "detail")
    assert "RLK_ERR_SHAPE" in str(err) and err.status == 3


def test_strided_layout_validation(lib):
    p = ctypes.c_void_p(16)
    R = rlk.RlkRows
    ok_rows = R(4, 40, 10)
    assert lib.rlk_entropy_fwd_strided(p, 1, 8, 10, None, F(0), p, p, None) == ARG
    assert lib.rlk_entropy_fwd_strided(p, 1, 8, 10, ctypes.byref(R(0, 40, 10)), F(0), p, p,
                                       None) == SHAPE
    assert lib.rlk_entropy_fwd_strided(p, 1, 8, 10, ctypes.byref(R(4, -1, 10)), F(0), p, p,
                                       None) == SHAPE
    # overlapping gradient rows are rejected; overlapping input rows are not
    bad_g = R(4, 40, 5)
    assert lib.rlk_entropy_bwd_strided(p, 1, 8, 10, ctypes.byref(ok_rows), F(0), p, p, p,
                                       ctypes.byref(bad_g), None) == SHAPE
    bcast = R(4, 0, 0)
    st = lib.rlk_entropy_bwd_strided(p, 1, 8, 10, ctypes.byref(bcast), F(0), p, p, p,
                                     ctypes.byref(ok_rows), None)
    assert st == DEVICE  # validation passed; the fake pointers fail at device binding
    # time-major gradient layout ([T, B, V] seen as [B, T, V]) is accepted
    tm = R(4, 10, 20)
    st = lib.rlk_logp_bwd_strided(p, 1, 8, 10, ctypes.byref(ok_rows), p, 1, F(0), p, p, p,
                                  ctypes.byref(tm), None)
    assert st == DEVICE
    assert lib.rlk_kl_fwd_strided(None, None, 1, 0, 10, None, None, 0, F(0), F(0), None, None,
                                  None) == ARG  # layout pointers are required even for N = 0


def test_shard_entry_points_validate(lib):
    p = ctypes.c_void_p(16)
    I64 = ctypes.c_int64
    assert lib.rlk_partial_bytes(5) == 160 and lib.rlk_partial_bytes(0) == 0
    # shard [v0, v0 + V_shard) must lie inside [0, V_total)
    assert lib.rlk_logp_fwd_partial(p, 1, 4, 8, 8, 10, 16, p, 1, F(0), p, p, None) == SHAPE
    assert lib.rlk_logp_fwd_partial(p, 1, 4, 8, 8, -1, 16, p, 1, F(0), p, p, None) == SHAPE
    assert lib.rlk_logp_fwd_partial(p, 1, 4, 8, 6, 0, 16, p, 1, F(0), p, p, None) == SHAPE
    assert lib.rlk_logp_fwd_partial(p, 1, 4, 8, 8, 0, 16, p, 0, F(0), p, p, None) == SHAPE
    assert lib.rlk_logp_fwd_partial(p, 1, 4, 8, 8, 0, 16, p, 1, F(0), p, None, None) == ARG
    assert lib.rlk_logp_fwd_partial(p, 1, 0, 8, 8, 0, 16, p, 1, F(0), p, p, None) == OK
    assert lib.rlk_entropy_fwd_partial(p, 1, 4, -1, 8, F(0), p, None) == SHAPE
    assert lib.rlk_entropy_fwd_partial(p, 1, 4, 8, 8, F(0), None, None) == ARG
    assert lib.rlk_kl_fwd_partial(p, p, 1, 4, 8, 8, 8, 3, F(0), F(0), p, None) == ARG
    assert lib.rlk_logp_bwd_shard(p, 1, 4, 8, 8, 12, 16, p, 1, F(0), p, p, p, None) == SHAPE
    assert lib.rlk_logp_bwd_shard(p, 1, 4, 0, 0, 16, 16, p, 1, F(0), p, p, p, None) == OK
    # combine: head, shard count, bounds
    b = (I64 * 3)(0, 5, 9)
    assert lib.rlk_combine(7, 0, 2, b, 4, p, p, 1, p, F(0), p, p, None) == ARG
    assert lib.rlk_combine(2, 5, 2, b, 4, p, p, 1, p, F(0), p, p, None) == ARG
    assert lib.rlk_combine(1, 0, 0, b, 4, p, p, 1, p, F(0), p, p, None) == SHAPE
    assert lib.rlk_combine(1, 0, 65, b, 4, p, p, 1, p, F(0), p, p, None) == SHAPE
    assert lib.rlk_combine(1, 0, 2, None, 4, p, p, 1, p, F(0), p, p, None) == ARG
    assert lib.rlk_combine(1, 0, 2, (I64 * 3)(1, 5, 9), 4, p, p, 1, p, F(0), p, p,
                           None) == SHAPE
    assert lib.rlk_combine(1, 0, 2, (I64 * 3)(0, 5, 4), 4, p, p, 1, p, F(0), p, p,
                           None) == SHAPE
    assert lib.rlk_combine(1, 0, 2, (I64 * 3)(0, 0, 0), 4, p, p, 1, p, F(0), p, p,
                           None) == SHAPE
    assert lib.rlk_combine(0, 0, 2, b, 4, p, None, 1, p, F(0), p, p, None) == ARG
    assert lib.rlk_combine(0, 0, 2, b, 4, p, p, 1, p, F(-1), p, p, None) == ARG
    assert lib.rlk_combine(1, 0, 2, b, 0, None, None, 1, None, F(0), None, None, None) == OK


def test_kl_both_and_reference_gradient_validate(lib):
    p = ctypes.c_void_p(16)
    # both directions: the forward-KL outputs are required
    assert lib.rlk_kl_fwd_both(p, p, 1, 4, 8, 8, 8, F(0), F(0), p, p, None, p, None) == ARG
    assert lib.rlk_kl_fwd_both(p, p, 1, 4, 8, 8, 8, F(0), F(0), p, p, p, None, None) == ARG
    assert lib.rlk_kl_fwd_both(p, p, 1, 4, 8, 7, 8, F(0), F(0), p, p, p, p, None) == SHAPE
    assert lib.rlk_kl_fwd_both(p, p, 3, 4, 8, 8, 8, F(0), F(0), p, p, p, p, None) == DTYPE
    assert lib.rlk_kl_fwd_both(p, p, 1, 0, 8, 8, 8, F(0), F(0), None, None, None, None,
                               None) == OK
    # reference gradient
    assert lib.rlk_kl_bwd_ref(p, p, 1, 4, 8, 8, 8, 2, F(0), F(0), p, p, p, None) == ARG
    assert lib.rlk_kl_bwd_ref(p, p, 1, 4, 8, 8, 6, 0, F(0), F(0), p, p, p, None) == SHAPE
    assert lib.rlk_kl_bwd_ref(p, p, 1, 4, 8, 8, 8, 0, F(0), F(-2), p, p, p, None) == ARG
    assert lib.rlk_kl_bwd_ref(p, p, 1, 4, 8, 8, 8, 0, F(0), F(0), p, p, None, None) == ARG
    R = rlk.RlkRows
    assert lib.rlk_kl_bwd_ref_strided(p, p, 1, 8, 10, ctypes.byref(R(4, 40, 10)),
                                      ctypes.byref(R(4, 40, 10)), 0, F(0), F(0), p, p, p,
                                      ctypes.byref(R(4, 20, 5)), None) == SHAPE


def test_missing_library_fails_loudly(tmp_path):
    # no fallback implementation: without librlk.so the binding refuses to load
    code = ("from vocab_log_softmax_amd import rlk\n"
            "try:\n"
            "    rlk.load_library()\n"
            "except ImportError as e:\n"
            "    print('ImportError:', e)\n"
            "    raise SystemExit(3)\n"
            "raise SystemExit(0)\n")
    env = dict(os.environ, RLK_LIB=str(tmp_path / "librlk.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 3, r.stdout + r.stderr
    assert "no fallback" in r.stdout


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr, r.stdout + r.stderr
