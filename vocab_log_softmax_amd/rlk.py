"""Python binding of the C ABI in ``include/rlk.h`` (argument marshalling only).

The functions below carry the C names (``rlk_logp_fwd`` ...).  They check torch
dtypes and shapes, pass raw device pointers, row strides and the current HIP
stream of the tensors' device, and raise ``RLKError`` on a non-OK status.
Every step of the computation runs in ``librlk.so``; there is no fallback: if
the library is missing, the import of the functions fails loudly.

Convenience layers (allocate outputs with torch, then call the same entry
points): ``logp_fwd`` / ``logp_bwd`` / ``entropy_fwd`` / ... and the autograd
functions ``logprobs``, ``entropy``, ``kl_divergence`` and ``softcap``.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("RLK_LIB", os.path.join(_PKG, "librlk.so"))

RLK_F32, RLK_BF16, RLK_F16 = 0, 1, 2
RLK_HEAD_LOGP, RLK_HEAD_ENTROPY, RLK_HEAD_KL = 0, 1, 2
RLK_KL_REVERSE, RLK_KL_FORWARD = 0, 1
RLK_MAX_TOPK = 4096
RLK_MAX_SHARDS = 64
STATUS = {0: "RLK_OK", 1: "RLK_ERR_ARG", 2: "RLK_ERR_DTYPE", 3: "RLK_ERR_SHAPE",
          4: "RLK_ERR_DEVICE", 5: "RLK_ERR_LAUNCH"}

EXPORTS = ("rlk_abi_version", "rlk_stats_bytes", "rlk_status_str", "rlk_last_error",
           "rlk_softcap_fwd", "rlk_softcap_bwd", "rlk_logp_fwd", "rlk_logp_bwd",
           "rlk_entropy_fwd", "rlk_entropy_bwd", "rlk_kl_fwd", "rlk_kl_bwd",
           "rlk_logp_fwd_strided", "rlk_logp_bwd_strided", "rlk_entropy_fwd_strided",
           "rlk_entropy_bwd_strided", "rlk_kl_fwd_strided", "rlk_kl_bwd_strided",
           "rlk_partial_bytes", "rlk_logp_fwd_partial", "rlk_entropy_fwd_partial",
           "rlk_kl_fwd_partial", "rlk_combine", "rlk_logp_bwd_shard", "rlk_kl_fwd_both",
           "rlk_kl_fwd_both_strided", "rlk_kl_bwd_ref", "rlk_kl_bwd_ref_strided")


class RlkRows(ctypes.Structure):
    """ctypes mirror of rlk_rows: row i = (i // T, i % T) at b*batch_stride + t*row_stride."""
    _fields_ = [("rows_per_batch", ctypes.c_int64), ("batch_stride", ctypes.c_int64),
                ("row_stride", ctypes.c_int64)]


class RLKError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load librlk.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i64, f32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    rp = ctypes.POINTER(RlkRows)
    sig = {
        "rlk_abi_version": ([], ci),
        "rlk_stats_bytes": ([ci, i64, i64], ctypes.c_size_t),
        "rlk_status_str": ([ci], ctypes.c_char_p),
        "rlk_last_error": ([], ctypes.c_char_p),
        "rlk_softcap_fwd": ([vp, ci, vp, ci, i64, f32, vp], ci),
        "rlk_softcap_bwd": ([vp, ci, vp, vp, i64, f32, vp], ci),
        "rlk_logp_fwd": ([vp, ci, i64, i64, i64, vp, i64, f32, vp, vp, vp], ci),
        "rlk_logp_bwd": ([vp, ci, i64, i64, i64, vp, i64, f32, vp, vp, vp, vp], ci),
        "rlk_entropy_fwd": ([vp, ci, i64, i64, i64, f32, vp, vp, vp], ci),
        "rlk_entropy_bwd": ([vp, ci, i64, i64, i64, f32, vp, vp, vp, vp], ci),
        "rlk_kl_fwd": ([vp, vp, ci, i64, i64, i64, i64, ci, f32, f32, vp, vp, vp], ci),
        "rlk_kl_bwd": ([vp, vp, ci, i64, i64, i64, i64, ci, f32, f32, vp, vp, vp, vp], ci),
        "rlk_logp_fwd_strided": ([vp, ci, i64, i64, rp, vp, i64, f32, vp, vp, vp], ci),
        "rlk_logp_bwd_strided": ([vp, ci, i64, i64, rp, vp, i64, f32, vp, vp, vp, rp, vp], ci),
        "rlk_entropy_fwd_strided": ([vp, ci, i64, i64, rp, f32, vp, vp, vp], ci),
        "rlk_entropy_bwd_strided": ([vp, ci, i64, i64, rp, f32, vp, vp, vp, rp, vp], ci),
        "rlk_kl_fwd_strided": ([vp, vp, ci, i64, i64, rp, rp, ci, f32, f32, vp, vp, vp], ci),
        "rlk_kl_bwd_strided": ([vp, vp, ci, i64, i64, rp, rp, ci, f32, f32, vp, vp, vp, rp,
                                vp], ci),
        "rlk_partial_bytes": ([i64], ctypes.c_size_t),
        "rlk_logp_fwd_partial": ([vp, ci, i64, i64, i64, i64, i64, vp, i64, f32, vp, vp, vp],
                                 ci),
        "rlk_entropy_fwd_partial": ([vp, ci, i64, i64, i64, f32, vp, vp], ci),
        "rlk_kl_fwd_partial": ([vp, vp, ci, i64, i64, i64, i64, ci, f32, f32, vp, vp], ci),
        "rlk_combine": ([ci, ci, i64, ctypes.POINTER(i64), i64, vp, vp, i64, vp, f32, vp, vp,
                         vp], ci),
        "rlk_logp_bwd_shard": ([vp, ci, i64, i64, i64, i64, i64, vp, i64, f32, vp, vp, vp, vp],
                               ci),
        "rlk_kl_fwd_both": ([vp, vp, ci, i64, i64, i64, i64, f32, f32, vp, vp, vp, vp, vp], ci),
        "rlk_kl_fwd_both_strided": ([vp, vp, ci, i64, i64, rp, rp, f32, f32, vp, vp, vp, vp, vp],
                                    ci),
        "rlk_kl_bwd_ref": ([vp, vp, ci, i64, i64, i64, i64, ci, f32, f32, vp, vp, vp, vp], ci),
        "rlk_kl_bwd_ref_strided": ([vp, vp, ci, i64, i64, rp, rp, ci, f32, f32, vp, vp, vp, rp,
                                    vp], ci),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


_prep = threading.local()


def _call(name: str, *args) -> None:
    rec = getattr(_prep, "calls", None)
    if rec is not None:            # inside prepare(): record instead of calling
        rec.append((name, args))
        return
    lib = load_library()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise RLKError(name, st, lib.rlk_last_error().decode())


def prepare(fn, *args, **kwargs):
    """Marshal one call of a raw binding function once; return a callable that
    repeats exactly that C call.

    ``fn`` is one of the ``rlk_*`` functions of this module and ``args`` its
    arguments.  The tensor checks, pointer and stream conversions are done
    here, once; each call of the result only enters the C library (which still
    validates every argument).  For tight loops over fixed buffers on the
    current stream, where those per-call conversions would cost more than a
    small kernel; the buffers must outlive the callable.
    """
    _prep.calls = []
    try:
        fn(*args, **kwargs)
        calls = _prep.calls
    finally:
        _prep.calls = None
    if len(calls) != 1:
        raise ValueError(f"{getattr(fn, '__name__', fn)} did not make exactly one library call")
    name, cargs = calls[0]
    lib = load_library()
    cfn = getattr(lib, name)
    keep = args  # the tensors whose pointers the call holds

    def call() -> None:
        st = cfn(*cargs)
        if st != 0:
            raise RLKError(name, st, lib.rlk_last_error().decode())

    call.tensors = keep
    return call


# ------------------------------------------------------------ marshalling

def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype == torch.float32:
        return RLK_F32
    if t.dtype == torch.bfloat16:
        return RLK_BF16
    if t.dtype == torch.float16:
        return RLK_F16
    raise TypeError(f"{what} must be float32, bfloat16 or float16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# torch's current HIP stream of a device as a raw handle; the private accessor
# skips building a Stream object (about 1.5 us per call), the public one is
# the fallback.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor):
    dev = t.device
    if dev.type != "cuda":
        raise ValueError(f"tensor must be on a GPU device, got {dev}")
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(idx))
    return ctypes.c_void_p(torch.cuda.current_stream(idx).cuda_stream)


def _rows(x: torch.Tensor, what: str) -> torch.Tensor:
    """2-D view whose vocabulary dimension is unit-stride (copy only if not)."""
    if x.dim() != 2:
        raise ValueError(f"{what} must be 2-D [N, V], got shape {tuple(x.shape)}")
    if x.stride(1) != 1 or x.stride(0) < x.shape[1]:
        x = x.contiguous()
    return x


def _view3(x: torch.Tensor, what: str) -> torch.Tensor:
    """[B, T, V] view with a unit-stride vocabulary dimension (copy only if not)."""
    if x.dim() != 3:
        raise ValueError(f"{what} must be 3-D [B, T, V], got shape {tuple(x.shape)}")
    if x.stride(2) != 1 and x.shape[2] > 1:
        x = x.contiguous()
    return x


def rows_of(x: torch.Tensor) -> RlkRows:
    """rlk_rows of a [B, T, V] (or [N, V]) view with unit-stride last dimension."""
    if x.dim() == 2:
        return RlkRows(max(1, x.shape[0]), 0, _ld(x))
    B, T, V = x.shape
    st = x.stride(1) if T > 1 else V
    sb = x.stride(0) if B > 1 else T * st
    return RlkRows(max(1, T), sb, st)


def _ld(x: torch.Tensor) -> int:
    return x.stride(0) if x.shape[0] > 1 else max(x.stride(0), x.shape[1])


def _need(t: torch.Tensor, dtype, shape, what: str):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def rlk_abi_version() -> int:
    return int(load_library().rlk_abi_version())


def rlk_stats_bytes(head: int, N: int, V: int) -> int:
    return int(load_library().rlk_stats_bytes(head, N, V))


def rlk_status_str(status: int) -> str:
    return load_library().rlk_status_str(status).decode()


def rlk_last_error() -> str:
    return load_library().rlk_last_error().decode()


def rlk_softcap_fwd(x: torch.Tensor, y: torch.Tensor, cap: float) -> None:
    if not x.is_contiguous() or not y.is_contiguous() or x.numel() != y.numel():
        raise ValueError("x and y must be contiguous with the same number of elements")
    _call("rlk_softcap_fwd", _ptr(x), _dtype_code(x, "x"), _ptr(y), _dtype_code(y, "y"),
          x.numel(), float(cap), _stream(x))


def rlk_softcap_bwd(x: torch.Tensor, grad_y: torch.Tensor, grad_x: torch.Tensor,
                    cap: float) -> None:
    _need(grad_y, torch.float32, x.shape, "grad_y")
    _need(grad_x, x.dtype, x.shape, "grad_x")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    _call("rlk_softcap_bwd", _ptr(x), _dtype_code(x, "x"), _ptr(grad_y), _ptr(grad_x),
          x.numel(), float(cap), _stream(x))


def rlk_logp_fwd(logits, targets, softcap, logp, stats) -> None:
    N, V = logits.shape
    k = targets.shape[1]
    _need(targets, torch.int64, (N, k), "targets")
    _need(logp, torch.float32, (N, k), "logp")
    _call("rlk_logp_fwd", _ptr(logits), _dtype_code(logits, "logits"), N, V, _ld(logits),
          _ptr(targets), k, float(softcap), _ptr(logp), _ptr(stats), _stream(logits))


def rlk_logp_bwd(logits, targets, softcap, stats, grad_logp, grad_logits) -> None:
    N, V = logits.shape
    k = targets.shape[1]
    _need(targets, torch.int64, (N, k), "targets")
    _need(grad_logp, torch.float32, (N, k), "grad_logp")
    _need(grad_logits, logits.dtype, (N, V), "grad_logits")
    _call("rlk_logp_bwd", _ptr(logits), _dtype_code(logits, "logits"), N, V, _ld(logits),
          _ptr(targets), k, float(softcap), _ptr(stats), _ptr(grad_logp), _ptr(grad_logits),
          _stream(logits))


def rlk_entropy_fwd(logits, softcap, entropy, stats) -> None:
    N, V = logits.shape
    _need(entropy, torch.float32, (N,), "entropy")
    _call("rlk_entropy_fwd", _ptr(logits), _dtype_code(logits, "logits"), N, V, _ld(logits),
          float(softcap), _ptr(entropy), _ptr(stats), _stream(logits))


def rlk_entropy_bwd(logits, softcap, stats, grad_entropy, grad_logits) -> None:
    N, V = logits.shape
    _need(grad_entropy, torch.float32, (N,), "grad_entropy")
    _need(grad_logits, logits.dtype, (N, V), "grad_logits")
    _call("rlk_entropy_bwd", _ptr(logits), _dtype_code(logits, "logits"), N, V, _ld(logits),
          float(softcap), _ptr(stats), _ptr(grad_entropy), _ptr(grad_logits), _stream(logits))


def rlk_kl_fwd(policy, ref, direction, softcap_policy, softcap_ref, kl, stats) -> None:
    N, V = policy.shape
    if tuple(ref.shape) != (N, V) or ref.dtype != policy.dtype:
        raise ValueError("policy and ref must have the same shape and dtype")
    _need(kl, torch.float32, (N,), "kl")
    _call("rlk_kl_fwd", _ptr(policy), _ptr(ref), _dtype_code(policy, "policy"), N, V,
          _ld(policy), _ld(ref), int(direction), float(softcap_policy), float(softcap_ref),
          _ptr(kl), _ptr(stats), _stream(policy))


def rlk_kl_bwd(policy, ref, direction, softcap_policy, softcap_ref, stats, grad_kl,
               grad_policy) -> None:
    N, V = policy.shape
    _need(grad_kl, torch.float32, (N,), "grad_kl")
    _need(grad_policy, policy.dtype, (N, V), "grad_policy")
    _call("rlk_kl_bwd", _ptr(policy), _ptr(ref), _dtype_code(policy, "policy"), N, V,
          _ld(policy), _ld(ref), int(direction), float(softcap_policy), float(softcap_ref),
          _ptr(stats), _ptr(grad_kl), _ptr(grad_policy), _stream(policy))


def rlk_kl_fwd_both(policy, ref, softcap_policy, softcap_ref, kl_rev, stats_rev, kl_fwd,
                    stats_fwd) -> None:
    N, V = policy.shape
    if tuple(ref.shape) != (N, V) or ref.dtype != policy.dtype:
        raise ValueError("policy and ref must have the same shape and dtype")
    _need(kl_rev, torch.float32, (N,), "kl_rev")
    _need(kl_fwd, torch.float32, (N,), "kl_fwd")
    _call("rlk_kl_fwd_both", _ptr(policy), _ptr(ref), _dtype_code(policy, "policy"), N, V,
          _ld(policy), _ld(ref), float(softcap_policy), float(softcap_ref), _ptr(kl_rev),
          _ptr(stats_rev), _ptr(kl_fwd), _ptr(stats_fwd), _stream(policy))


def rlk_kl_bwd_ref(policy, ref, direction, softcap_policy, softcap_ref, stats, grad_kl,
                   grad_ref) -> None:
    N, V = policy.shape
    _need(grad_kl, torch.float32, (N,), "grad_kl")
    _need(grad_ref, ref.dtype, (N, V), "grad_ref")
    _call("rlk_kl_bwd_ref", _ptr(policy), _ptr(ref), _dtype_code(policy, "policy"), N, V,
          _ld(policy), _ld(ref), int(direction), float(softcap_policy), float(softcap_ref),
          _ptr(stats), _ptr(grad_kl), _ptr(grad_ref), _stream(policy))


def rlk_kl_fwd_both_strided(policy, ref, softcap_policy, softcap_ref, kl_rev, stats_rev, kl_fwd,
                            stats_fwd) -> None:
    B, T, V = policy.shape
    N = B * T
    _need(kl_rev, torch.float32, (N,), "kl_rev")
    _need(kl_fwd, torch.float32, (N,), "kl_fwd")
    rp, rr = rows_of(policy), rows_of(ref)
    _call("rlk_kl_fwd_both_strided", _ptr(policy), _ptr(ref), _dtype_code(policy, "policy"), N,
          V, ctypes.byref(rp), ctypes.byref(rr), float(softcap_policy), float(softcap_ref),
          _ptr(kl_rev), _ptr(stats_rev), _ptr(kl_fwd), _ptr(stats_fwd), _stream(policy))


def rlk_kl_bwd_ref_strided(policy, ref, direction, softcap_policy, softcap_ref, stats, grad_kl,
                           grad_ref) -> None:
    B, T, V = policy.shape
    N = B * T
    _need(grad_kl, torch.float32, (N,), "grad_kl")
    if grad_ref.dtype != ref.dtype or tuple(grad_ref.shape) != (B, T, V):
        raise ValueError("grad_ref must be a [B, T, V] view in the logits dtype")
    rp, rr, rg = rows_of(policy), rows_of(ref), rows_of(grad_ref)
    _call("rlk_kl_bwd_ref_strided", _ptr(policy), _ptr(ref), _dtype_code(policy, "policy"), N,
          V, ctypes.byref(rp), ctypes.byref(rr), int(direction), float(softcap_policy),
          float(softcap_ref), _ptr(stats), _ptr(grad_kl), _ptr(grad_ref), ctypes.byref(rg),
          _stream(policy))


def rlk_logp_fwd_strided(logits, targets, softcap, logp, stats) -> None:
    B, T, V = logits.shape
    N, k = B * T, targets.shape[-1]
    _need(targets, torch.int64, (N, k), "targets")
    _need(logp, torch.float32, (N, k), "logp")
    r = rows_of(logits)
    _call("rlk_logp_fwd_strided", _ptr(logits), _dtype_code(logits, "logits"), N, V,
          ctypes.byref(r), _ptr(targets), k, float(softcap), _ptr(logp), _ptr(stats),
          _stream(logits))


def rlk_logp_bwd_strided(logits, targets, softcap, stats, grad_logp, grad_logits) -> None:
    B, T, V = logits.shape
    N, k = B * T, targets.shape[-1]
    _need(targets, torch.int64, (N, k), "targets")
    _need(grad_logp, torch.float32, (N, k), "grad_logp")
    if grad_logits.dtype != logits.dtype or tuple(grad_logits.shape) != (B, T, V):
        raise ValueError("grad_logits must be a [B, T, V] view in the logits dtype")
    r, rg = rows_of(logits), rows_of(grad_logits)
    _call("rlk_logp_bwd_strided", _ptr(logits), _dtype_code(logits, "logits"), N, V,
          ctypes.byref(r), _ptr(targets), k, float(softcap), _ptr(stats), _ptr(grad_logp),
          _ptr(grad_logits), ctypes.byref(rg), _stream(logits))


def rlk_entropy_fwd_strided(logits, softcap, entropy, stats) -> None:
    B, T, V = logits.shape
    _need(entropy, torch.float32, (B * T,), "entropy")
    r = rows_of(logits)
    _call("rlk_entropy_fwd_strided", _ptr(logits), _dtype_code(logits, "logits"), B * T, V,
          ctypes.byref(r), float(softcap), _ptr(entropy), _ptr(stats), _stream(logits))


def rlk_entropy_bwd_strided(logits, softcap, stats, grad_entropy, grad_logits) -> None:
    B, T, V = logits.shape
    _need(grad_entropy, torch.float32, (B * T,), "grad_entropy")
    if grad_logits.dtype != logits.dtype or tuple(grad_logits.shape) != (B, T, V):
        raise ValueError("grad_logits must be a [B, T, V] view in the logits dtype")
    r, rg = rows_of(logits), rows_of(grad_logits)
    _call("rlk_entropy_bwd_strided", _ptr(logits), _dtype_code(logits, "logits"), B * T, V,
          ctypes.byref(r), float(softcap), _ptr(stats), _ptr(grad_entropy), _ptr(grad_logits),
          ctypes.byref(rg), _stream(logits))


def rlk_kl_fwd_strided(policy, ref, direction, softcap_policy, softcap_ref, kl, stats) -> None:
    B, T, V = policy.shape
    if tuple(ref.shape) != (B, T, V) or ref.dtype != policy.dtype:
        raise ValueError("policy and ref must have the same shape and dtype")
    _need(kl, torch.float32, (B * T,), "kl")
    rp, rr = rows_of(policy), rows_of(ref)
    _call("rlk_kl_fwd_strided", _ptr(policy), _ptr(ref), _dtype_code(policy, "policy"), B * T, V,
          ctypes.byref(rp), ctypes.byref(rr), int(direction), float(softcap_policy),
          float(softcap_ref), _ptr(kl), _ptr(stats), _stream(policy))


def rlk_kl_bwd_strided(policy, ref, direction, softcap_policy, softcap_ref, stats, grad_kl,
                       grad_policy) -> None:
    B, T, V = policy.shape
    _need(grad_kl, torch.float32, (B * T,), "grad_kl")
    if grad_policy.dtype != policy.dtype or tuple(grad_policy.shape) != (B, T, V):
        raise ValueError("grad_policy must be a [B, T, V] view in the logits dtype")
    rp, rr, rg = rows_of(policy), rows_of(ref), rows_of(grad_policy)
    _call("rlk_kl_bwd_strided", _ptr(policy), _ptr(ref), _dtype_code(policy, "policy"), B * T, V,
          ctypes.byref(rp), ctypes.byref(rr), int(direction), float(softcap_policy),
          float(softcap_ref), _ptr(stats), _ptr(grad_kl), _ptr(grad_policy), ctypes.byref(rg),
          _stream(policy))


# ------------------------------------------------------- vocabulary shards
# A shard is the [N, V_shard] block of columns [v0, v0 + V_shard) of rows of
# width V_total (a 2-D view with unit column stride; V_shard may be 0).

def _shard(x: torch.Tensor, what: str):
    if x.dim() != 2:
        raise ValueError(f"{what} must be 2-D [N, V_shard], got shape {tuple(x.shape)}")
    N, Vs = x.shape
    if Vs > 0 and (x.stride(1) != 1 or (N > 1 and x.stride(0) < Vs)):
        raise ValueError(f"{what} must have unit column stride and row stride >= V_shard")
    ld = _ld(x) if Vs > 0 else 0
    return N, Vs, ld


def rlk_partial_bytes(N: int) -> int:
    return load_library().rlk_partial_bytes(N)


def rlk_logp_fwd_partial(logits, v0, V_total, targets, softcap, partial, target_vals) -> None:
    N, Vs, ld = _shard(logits, "logits")
    k = targets.shape[1]
    _need(targets, torch.int64, (N, k), "targets")
    _need(target_vals, torch.float32, (N, k), "target_vals")
    _call("rlk_logp_fwd_partial", _ptr(logits) if Vs else None, _dtype_code(logits, "logits"),
          N, Vs, ld, int(v0), int(V_total), _ptr(targets), k, float(softcap), _ptr(partial),
          _ptr(target_vals), _stream(targets))


def rlk_entropy_fwd_partial(logits, softcap, partial) -> None:
    N, Vs, ld = _shard(logits, "logits")
    _call("rlk_entropy_fwd_partial", _ptr(logits) if Vs else None,
          _dtype_code(logits, "logits"), N, Vs, ld, float(softcap), _ptr(partial),
          _stream(partial))


def rlk_kl_fwd_partial(policy, ref, direction, softcap_policy, softcap_ref, partial) -> None:
    N, Vs, ldp = _shard(policy, "policy")
    if tuple(ref.shape) != (N, Vs) or ref.dtype != policy.dtype:
        raise ValueError("policy and ref shards must have the same shape and dtype")
    _, _, ldr = _shard(ref, "ref")
    _call("rlk_kl_fwd_partial", _ptr(policy) if Vs else None, _ptr(ref) if Vs else None,
          _dtype_code(policy, "policy"), N, Vs, ldp, ldr, int(direction),
          float(softcap_policy), float(softcap_ref), _ptr(partial), _stream(partial))


def rlk_combine(head, direction, bounds, partials, targets, target_vals, softcap, out,
                stats) -> None:
    """Fold gathered shard records partials [P, N * 32 bytes] in rank order."""
    P = len(bounds) - 1
    b = (ctypes.c_int64 * (P + 1))(*[int(v) for v in bounds])
    N = out.shape[0]
    k = targets.shape[1] if targets is not None else 1
    if head == RLK_HEAD_LOGP:
        _need(targets, torch.int64, (N, k), "targets")
        _need(target_vals, torch.float32, (P, N, k), "target_vals")
        _need(out, torch.float32, (N, k), "out")
    else:
        _need(out, torch.float32, (N,), "out")
    _call("rlk_combine", int(head), int(direction), P, b, N, _ptr(partials), _ptr(targets), k,
          _ptr(target_vals), float(softcap), _ptr(out), _ptr(stats), _stream(out))


def rlk_logp_bwd_shard(logits, v0, V_total, targets, softcap, stats, grad_logp,
                       grad_logits) -> None:
    N, Vs, ld = _shard(logits, "logits")
    k = targets.shape[1]
    _need(targets, torch.int64, (N, k), "targets")
    _need(grad_logp, torch.float32, (N, k), "grad_logp")
    _need(grad_logits, logits.dtype, (N, Vs), "grad_logits")
    _call("rlk_logp_bwd_shard", _ptr(logits) if Vs else None, _dtype_code(logits, "logits"), N,
          Vs, ld, int(v0), int(V_total), _ptr(targets), k, float(softcap), _ptr(stats),
          _ptr(grad_logp), _ptr(grad_logits), _stream(targets))


def new_partials(P: int, N: int, device) -> torch.Tensor:
    """Uninitialised buffer for P shard records of N rows ([P, N * 32] bytes)."""
    return torch.empty((P, max(1, rlk_partial_bytes(N))), dtype=torch.uint8, device=device)


# ------------------------------------------------ allocating convenience layer

def new_stats(head: int, N: int, V: int, device) -> torch.Tensor:
    return torch.empty(max(1, rlk_stats_bytes(head, N, V)), dtype=torch.uint8, device=device)


def _targets2d(targets: torch.Tensor, N: int) -> torch.Tensor:
    t = targets.reshape(N, -1)
    return t.contiguous() if t.dtype == torch.int64 else t.to(torch.int64).contiguous()


# The allocating wrappers accept [N, V] matrices and [B, T, V] views (read in
# place, e.g. logits[:, :-1]); outputs are [N] / [N, k] (or [B, T] / [B, T, k])
# and gradients come back contiguous in the input's shape.

def logp_fwd(logits, targets, softcap=0.0):
    if logits.dim() == 3:
        logits = _view3(logits, "logits")
        B, T, V = logits.shape
        t = _targets2d(targets, B * T)
        out = torch.empty(t.shape, dtype=torch.float32, device=logits.device)
        stats = new_stats(RLK_HEAD_LOGP, B * T, V, logits.device)
        rlk_logp_fwd_strided(logits, t, softcap, out, stats)
        return out.reshape(targets.shape), stats
    logits = _rows(logits, "logits")
    N, V = logits.shape
    t = _targets2d(targets, N)
    out = torch.empty(t.shape, dtype=torch.float32, device=logits.device)
    stats = new_stats(RLK_HEAD_LOGP, N, V, logits.device)
    rlk_logp_fwd(logits, t, softcap, out, stats)
    return out.reshape(targets.shape), stats


def logp_bwd(logits, targets, grad_logp, stats, softcap=0.0, out=None):
    """Gradient w.r.t. the logits; ``out`` may be a [B, T, V] view to write into."""
    if logits.dim() == 3:
        logits = _view3(logits, "logits")
        B, T, V = logits.shape
        t = _targets2d(targets, B * T)
        g = grad_logp.reshape(t.shape).to(torch.float32).contiguous()
        gx = out if out is not None else torch.empty((B, T, V), dtype=logits.dtype,
                                                     device=logits.device)
        rlk_logp_bwd_strided(logits, t, softcap, stats, g, gx)
        return gx
    logits = _rows(logits, "logits")
    N, V = logits.shape
    t = _targets2d(targets, N)
    g = grad_logp.reshape(t.shape).to(torch.float32).contiguous()
    gx = torch.empty((N, V), dtype=logits.dtype, device=logits.device)
    rlk_logp_bwd(logits, t, softcap, stats, g, gx)
    return gx


def entropy_fwd(logits, softcap=0.0):
    if logits.dim() == 3:
        logits = _view3(logits, "logits")
        B, T, V = logits.shape
        out = torch.empty(B * T, dtype=torch.float32, device=logits.device)
        stats = new_stats(RLK_HEAD_ENTROPY, B * T, V, logits.device)
        rlk_entropy_fwd_strided(logits, softcap, out, stats)
        return out.reshape(B, T), stats
    logits = _rows(logits, "logits")
    N, V = logits.shape
    out = torch.empty(N, dtype=torch.float32, device=logits.device)
    stats = new_stats(RLK_HEAD_ENTROPY, N, V, logits.device)
    rlk_entropy_fwd(logits, softcap, out, stats)
    return out, stats


def entropy_bwd(logits, grad_entropy, stats, softcap=0.0, out=None):
    if logits.dim() == 3:
        logits = _view3(logits, "logits")
        B, T, V = logits.shape
        gx = out if out is not None else torch.empty((B, T, V), dtype=logits.dtype,
                                                     device=logits.device)
        rlk_entropy_bwd_strided(logits, softcap, stats,
                                grad_entropy.reshape(-1).to(torch.float32).contiguous(), gx)
        return gx
    logits = _rows(logits, "logits")
    N, V = logits.shape
    gx = torch.empty((N, V), dtype=logits.dtype, device=logits.device)
    rlk_entropy_bwd(logits, softcap, stats, grad_entropy.to(torch.float32).contiguous(), gx)
    return gx


def kl_fwd(policy, ref, direction=RLK_KL_REVERSE, softcap_policy=0.0, softcap_ref=0.0):
    if policy.dim() == 3:
        policy, ref = _view3(policy, "policy"), _view3(ref, "ref")
        B, T, V = policy.shape
        out = torch.empty(B * T, dtype=torch.float32, device=policy.device)
        stats = new_stats(RLK_HEAD_KL, B * T, V, policy.device)
        rlk_kl_fwd_strided(policy, ref, direction, softcap_policy, softcap_ref, out, stats)
        return out.reshape(B, T), stats
    policy, ref = _rows(policy, "policy"), _rows(ref, "ref")
    N, V = policy.shape
    out = torch.empty(N, dtype=torch.float32, device=policy.device)
    stats = new_stats(RLK_HEAD_KL, N, V, policy.device)
    rlk_kl_fwd(policy, ref, direction, softcap_policy, softcap_ref, out, stats)
    return out, stats


def kl_bwd(policy, ref, grad_kl, stats, direction=RLK_KL_REVERSE, softcap_policy=0.0,
           softcap_ref=0.0, out=None):
    if policy.dim() == 3:
        policy, ref = _view3(policy, "policy"), _view3(ref, "ref")
        B, T, V = policy.shape
        gx = out if out is not None else torch.empty((B, T, V), dtype=policy.dtype,
                                                     device=policy.device)
        rlk_kl_bwd_strided(policy, ref, direction, softcap_policy, softcap_ref, stats,
                           grad_kl.reshape(-1).to(torch.float32).contiguous(), gx)
        return gx
    policy, ref = _rows(policy, "policy"), _rows(ref, "ref")
    N, V = policy.shape
    gx = torch.empty((N, V), dtype=policy.dtype, device=policy.device)
    rlk_kl_bwd(policy, ref, direction, softcap_policy, softcap_ref, stats,
               grad_kl.to(torch.float32).contiguous(), gx)
    return gx


def kl_fwd_both(policy, ref, softcap_policy=0.0, softcap_ref=0.0):
    """Reverse and forward KL from one read: (kl_rev, stats_rev, kl_fwd, stats_fwd)."""
    three = policy.dim() == 3
    if three:
        policy, ref = _view3(policy, "policy"), _view3(ref, "ref")
        B, T, V = policy.shape
        N = B * T
    else:
        policy, ref = _rows(policy, "policy"), _rows(ref, "ref")
        N, V = policy.shape
    outs = [torch.empty(N, dtype=torch.float32, device=policy.device) for _ in range(2)]
    sts = [new_stats(RLK_HEAD_KL, N, V, policy.device) for _ in range(2)]
    fn = rlk_kl_fwd_both_strided if three else rlk_kl_fwd_both
    fn(policy, ref, softcap_policy, softcap_ref, outs[0], sts[0], outs[1], sts[1])
    if three:
        outs = [o.reshape(B, T) for o in outs]
    return outs[0], sts[0], outs[1], sts[1]


def kl_bwd_ref(policy, ref, grad_kl, stats, direction=RLK_KL_REVERSE, softcap_policy=0.0,
               softcap_ref=0.0, out=None):
    """Gradient of the KL with respect to the reference logits."""
    if policy.dim() == 3:
        policy, ref = _view3(policy, "policy"), _view3(ref, "ref")
        B, T, V = policy.shape
        gr = out if out is not None else torch.empty((B, T, V), dtype=ref.dtype,
                                                     device=ref.device)
        rlk_kl_bwd_ref_strided(policy, ref, direction, softcap_policy, softcap_ref, stats,
                               grad_kl.reshape(-1).to(torch.float32).contiguous(), gr)
        return gr
    policy, ref = _rows(policy, "policy"), _rows(ref, "ref")
    N, V = policy.shape
    gr = torch.empty((N, V), dtype=ref.dtype, device=ref.device)
    rlk_kl_bwd_ref(policy, ref, direction, softcap_policy, softcap_ref, stats,
                   grad_kl.to(torch.float32).contiguous(), gr)
    return gr


def softcap_fwd(x, cap=30.0, out_dtype=torch.float32):
    x = x.contiguous()
    y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    rlk_softcap_fwd(x, y, cap)
    return y


def softcap_bwd(x, grad_y, cap=30.0):
    x = x.contiguous()
    gx = torch.empty_like(x)
    rlk_softcap_bwd(x, grad_y.to(torch.float32).contiguous(), gx, cap)
    return gx


# ------------------------------------------------------------------ autograd

class _LogProbs(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, targets, softcap):
        out, stats = logp_fwd(logits, targets, softcap)
        ctx.save_for_backward(logits, targets, stats)
        ctx.softcap = softcap
        return out

    @staticmethod
    def backward(ctx, g):
        logits, targets, stats = ctx.saved_tensors
        gx = logp_bwd(logits, targets, g, stats, ctx.softcap)
        return gx.reshape(logits.shape), None, None


class _Entropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, softcap):
        out, stats = entropy_fwd(logits, softcap)
        ctx.save_for_backward(logits, stats)
        ctx.softcap = softcap
        return out

    @staticmethod
    def backward(ctx, g):
        logits, stats = ctx.saved_tensors
        return entropy_bwd(logits, g, stats, ctx.softcap), None


class _KL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, policy, ref, direction, cp, cr):
        out, stats = kl_fwd(policy, ref, direction, cp, cr)
        ctx.save_for_backward(policy, ref, stats)
        ctx.args = (direction, cp, cr)
        return out

    @staticmethod
    def backward(ctx, g):
        policy, ref, stats = ctx.saved_tensors
        direction, cp, cr = ctx.args
        gp = kl_bwd(policy, ref, g, stats, direction, cp, cr) if ctx.needs_input_grad[0] else None
        gr = (kl_bwd_ref(policy, ref, g, stats, direction, cp, cr) if ctx.needs_input_grad[1]
              else None)
        return gp, gr, None, None, None


class _Softcap(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, cap):
        ctx.save_for_backward(x)
        ctx.cap = cap
        return softcap_fwd(x, cap)

    @staticmethod
    def backward(ctx, g):
        (x,) = ctx.saved_tensors
        return softcap_bwd(x, g, ctx.cap), None


def logprobs(logits, targets, softcap=0.0):
    """log softmax(softcap(logits))[targets] per row; ignored targets give 0."""
    return _LogProbs.apply(logits, targets, softcap)


def entropy(logits, softcap=0.0):
    return _Entropy.apply(logits, softcap)


def kl_divergence(policy, ref, direction=RLK_KL_REVERSE, softcap_policy=0.0, softcap_ref=0.0,
                  detach_ref=True):
    """KL per row; the gradient flows to ``policy`` and, with ``detach_ref=False``,
    to ``ref`` as well."""
    return _KL.apply(policy, ref.detach() if detach_ref else ref, direction, softcap_policy,
                     softcap_ref)


def softcap(x, cap=30.0):
    return _Softcap.apply(x, cap)
