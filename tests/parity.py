"""Comparison rules between the HIP path and the fp64 oracle.

Tolerances (fixed for this library; the reason for each is given with it):
  * head outputs (fp32) from fp32 logits: |d| <= 1e-5 + 1e-5 |ref|
    (relative 1e-5, with the 1e-5 absolute floor of the fp32 row of the
    accuracy table on the "Final Logit Softcap" page);
  * head outputs (fp32) from bf16 logits: |d| <= 2e-3;
  * fp32 gradients: |d| <= 1e-5 + 1e-5 |ref|;
  * bf16 gradients: |d| <= max(4e-3, one bf16 ulp of ref): a correct fp32
    value rounded once to bf16 is within half an ulp, and above |2| half an
    ulp already exceeds 4e-3;
  * fp16 logits: head outputs as for fp32 logits (the inputs are exact, the
    arithmetic is the same fp32); fp16 gradients |d| <= 1e-3 + 1e-3 |ref|
    (the fp16 row of the same accuracy table; half an fp16 ulp is 4.9e-4
    relative);
  * exact: the class of every element (NaN / +inf / -inf / finite) must
    match, and structural zeros (ignored targets, rows without a valid
    target, masked columns of entropy and reverse KL) must be exactly 0.
"""

from __future__ import annotations

import numpy as np
import torch

OUT_F32 = (1e-5, 1e-5)    # (abs, rel) for outputs from fp32 logits
OUT_BF16 = 2e-3
GRAD_F32 = (1e-5, 1e-5)
GRAD_BF16 = 4e-3
GRAD_F16 = (1e-3, 1e-3)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def bf16_ulp(r: np.ndarray) -> np.ndarray:
    a = np.abs(r).astype(np.float32)
    return np.spacing(a).astype(np.float64) * 65536.0


def _classes(a):
    return np.where(np.isnan(a), 3, np.where(np.isposinf(a), 1, np.where(np.isneginf(a), 2, 0)))


def assert_same_class(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    cg, cr = _classes(gpu), _classes(ref)
    bad = cg != cr
    if bad.any():
        idx = np.argwhere(bad)[:8]
        raise AssertionError(f"{what}: {bad.sum()} elements differ in NaN/inf class, e.g. "
                             + ", ".join(f"{tuple(i)} gpu={gpu[tuple(i)]} ref={ref[tuple(i)]}"
                                         for i in idx))


def _report(err, tol, gpu, ref, what):
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - tol, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance; "
                             f"worst at {i}: gpu={gpu[i]!r} ref={ref[i]!r} err={err[i]:.3g} "
                             f"tol={np.broadcast_to(tol, err.shape)[i]:.3g}")


def assert_out(gpu_t: torch.Tensor, ref: np.ndarray, in_dtype, what="out", exact_zero=None):
    gpu = to64(gpu_t)
    ref = np.asarray(ref, dtype=np.float64).reshape(gpu.shape)
    assert_same_class(gpu, ref, what)
    if exact_zero is not None:
        ez = np.asarray(exact_zero).reshape(gpu.shape)
        assert (gpu[ez] == 0).all(), f"{what}: structural zeros are not exactly 0"
    fin = np.isfinite(ref)
    with np.errstate(invalid="ignore"):   # inf - inf where both are infinite
        err = np.where(fin, np.abs(gpu - ref), 0.0)
    if in_dtype in (torch.float32, torch.float16):
        tol = OUT_F32[0] + OUT_F32[1] * np.abs(np.where(fin, ref, 0.0))
    else:
        tol = np.full(err.shape, OUT_BF16)
    _report(err, tol, gpu, ref, what)


def assert_grad(gpu_t: torch.Tensor, ref: np.ndarray, what="grad", exact_zero=None):
    gpu = to64(gpu_t)
    ref = np.asarray(ref, dtype=np.float64).reshape(gpu.shape)
    assert_same_class(gpu, ref, what)
    if exact_zero is not None:
        ez = np.asarray(exact_zero).reshape(gpu.shape)
        assert (gpu[ez] == 0).all(), f"{what}: structural zeros are not exactly 0"
    fin = np.isfinite(ref)
    r0 = np.where(fin, ref, 0.0)
    with np.errstate(invalid="ignore"):   # inf - inf where both are infinite
        err = np.where(fin, np.abs(gpu - ref), 0.0)
    if gpu_t.dtype == torch.float32:
        tol = GRAD_F32[0] + GRAD_F32[1] * np.abs(r0)
    elif gpu_t.dtype == torch.float16:
        tol = GRAD_F16[0] + GRAD_F16[1] * np.abs(r0)
    else:
        tol = np.maximum(GRAD_BF16, bf16_ulp(r0))
    _report(err, tol, gpu, ref, what)


def strict_bf16_misses(gpu_t: torch.Tensor, ref: np.ndarray) -> int:
    """How many finite bf16 gradient elements miss the strict 4e-3 bound."""
    gpu = to64(gpu_t)
    ref = np.asarray(ref, dtype=np.float64).reshape(gpu.shape)
    fin = np.isfinite(ref)
    return int((np.abs(gpu[fin] - ref[fin]) > GRAD_BF16).sum())
