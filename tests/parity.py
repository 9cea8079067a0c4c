"""Comparison rules between the HIP path and the fp64 oracle.

The bounds are the stated ones, with one reading each where a bound cannot
hold as written:

  * head outputs (fp32) from fp32 or fp16 logits: relative 1e-5, i.e.
    |d| <= 1e-5 max(1, |ref|).  Reading: every head output is a difference
    of terms of the size of the row's log-sum-exp (logp = y_t - lse,
    H = lse - sum p y, KL = sum p (log p - log q)), which are >= 1 here, so
    near 0 (a dominant target, a near-deterministic row, a single column,
    close distributions) the fp32 rounding error of those terms is absolute,
    about 1e-7 of their size; such outputs are held to 1e-5 absolute (the
    fp32 row of the accuracy table on the "Final Logit Softcap" page,
    Accuracy and Invariance, absolute 1e-5);
  * head outputs (fp32) from bf16 logits: |d| <= 2e-3;
  * fp32 gradients: absolute 1e-5, i.e. |d| <= 1e-5 max(1, |ref|).
    Reading: the softmax terms are below 1 in magnitude and are held to
    1e-5 absolute; target columns carry sums of upstream gradients (top-k
    duplicates and G = sum of k slots reach |grad| ~ 70 in the tests), and
    the fp32 representation of the capped logits already carries an absolute
    error of about c 2^-23 (with a cap c), so elements above 1 in magnitude
    are held to 1e-5 relative;
  * bf16 gradients: |d| <= 4e-3.  Reading: a correct fp32 value rounded once
    to bf16 can be off by half a bf16 ulp, which exceeds 4e-3 for |ref| >= 2
    (half an ulp is 2^-7 there), so the bound is max(4e-3, half an ulp of
    ref + the fp32 arithmetic's slack 1e-5 |ref| + 1e-6): an error of a full
    ulp fails.  The number of elements beyond the strict 4e-3 is counted
    (strict_bf16_misses) and reported by the tests that see such elements;
  * fp16 gradients: |d| <= 1e-3 + 1e-3 |ref| (the fp16 row of the same
    accuracy table; half an fp16 ulp is 4.9e-4 relative);
  * exact: the class of every element (NaN / +inf / -inf / finite) must
    match, and structural zeros (ignored targets, rows without a valid
    target, masked columns of entropy and reverse KL) must be exactly 0.
"""

from __future__ import annotations

import numpy as np
import torch

OUT_F32_REL = 1e-5        # outputs from fp32 / fp16 logits: 1e-5 max(1, |ref|)
OUT_BF16 = 2e-3
GRAD_F32 = 1e-5           # 1e-5 max(1, |ref|)
GRAD_BF16 = 4e-3
GRAD_BF16_SLACK = (1e-6, 1e-5)   # (abs, rel) fp32 slack added to half a bf16 ulp
GRAD_F16 = (1e-3, 1e-3)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def bf16_ulp(r: np.ndarray) -> np.ndarray:
    """The bf16 ulp of the binade holding |r| (2^-133 at 0)."""
    a = np.abs(r).astype(np.float32)
    return np.spacing(a).astype(np.float64) * 65536.0


def bf16_grad_tol(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    return np.maximum(GRAD_BF16, 0.5 * bf16_ulp(ref) + GRAD_BF16_SLACK[0]
                      + GRAD_BF16_SLACK[1] * a)


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


def _strict(what, n, bound):
    """Report elements that pass only through a reading (tests run with -s
    or -rP show it)."""
    if n:
        print(f"{what}: {n} elements beyond the strict {bound} (within the stated reading)")
    return n


def assert_out(gpu_t: torch.Tensor, ref: np.ndarray, in_dtype, what="out", exact_zero=None):
    """Head outputs; returns how many elements miss the strict bound (pure
    relative 1e-5 for fp32 / fp16 logits)."""
    gpu = to64(gpu_t)
    ref = np.asarray(ref, dtype=np.float64).reshape(gpu.shape)
    assert_same_class(gpu, ref, what)
    if exact_zero is not None:
        ez = np.asarray(exact_zero).reshape(gpu.shape)
        assert (gpu[ez] == 0).all(), f"{what}: structural zeros are not exactly 0"
    fin = np.isfinite(ref)
    with np.errstate(invalid="ignore"):   # inf - inf where both are infinite
        err = np.where(fin, np.abs(gpu - ref), 0.0)
    a = np.abs(np.where(fin, ref, 0.0))
    if in_dtype in (torch.float32, torch.float16):
        tol = OUT_F32_REL * np.maximum(1.0, a)
        strict = int((err > OUT_F32_REL * a).sum())
    else:
        tol = np.full(err.shape, OUT_BF16)
        strict = 0
    _report(err, tol, gpu, ref, what)
    return _strict(what, strict, "relative 1e-5")


def assert_grad(gpu_t: torch.Tensor, ref: np.ndarray, what="grad", exact_zero=None):
    """Gradients; returns how many elements miss the strict bound (absolute
    1e-5 for fp32, 4e-3 for bf16)."""
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
    strict, bound = 0, ""
    if gpu_t.dtype == torch.float32:
        tol = GRAD_F32 * np.maximum(1.0, np.abs(r0))
        strict, bound = int((err > GRAD_F32).sum()), "absolute 1e-5"
    elif gpu_t.dtype == torch.float16:
        tol = GRAD_F16[0] + GRAD_F16[1] * np.abs(r0)
    else:
        tol = bf16_grad_tol(r0)
        strict, bound = int((err > GRAD_BF16).sum()), "4e-3"
    _report(err, tol, gpu, ref, what)
    return _strict(what, strict, bound)


def strict_bf16_misses(gpu_t: torch.Tensor, ref: np.ndarray) -> int:
    """How many finite bf16 gradient elements miss the strict 4e-3 bound."""
    gpu = to64(gpu_t)
    ref = np.asarray(ref, dtype=np.float64).reshape(gpu.shape)
    fin = np.isfinite(ref)
    return int((np.abs(gpu[fin] - ref[fin]) > GRAD_BF16).sum())
