"""Fit the small-argument tanh polynomial used by the standalone softcap kernel.

tanh(u) = u + u^3 P(u^2) on |u| < 0.55, P of degree 4 (five coefficients).
The fit minimises the relative error of tanh with an iteratively reweighted
least-squares pass (weights grow where the error is largest, approaching a
minimax fit), then checks the fp32 Horner evaluation on a dense grid.

Prints the coefficients (c1 .. c5 for u^3 .. u^11) and the maximum relative
error; rlk_device.h (tanh_precise) holds the printed values.
"""

import numpy as np

BOUND = 0.55
DEGREE = 5


def fit(bound=BOUND, degree=DEGREE, iters=200):
    u = np.cos(np.linspace(0.0, np.pi / 2, 4000)) * bound + 1e-6
    w = u * u
    target = (np.tanh(u) - u) / u ** 3
    weight = w / (np.tanh(u) / u)   # relative error of tanh ~ u^2 * error of P
    A = np.vander(w, degree, increasing=True)
    c, *_ = np.linalg.lstsq(A * weight[:, None], target * weight, rcond=None)
    for _ in range(iters):
        r = (A @ c - target) * weight
        rw = 1.0 + 50.0 * (np.abs(r) / np.abs(r).max()) ** 2
        c, *_ = np.linalg.lstsq(A * (weight * rw)[:, None], target * weight * rw, rcond=None)
    return c


def max_rel_error_fp32(c, bound=BOUND):
    uu = np.linspace(1e-4, bound, 200001).astype(np.float32)
    u2 = (uu * uu).astype(np.float32)
    p = np.float32(c[-1])
    for cc in c[-2::-1]:
        p = (p * u2 + np.float32(cc)).astype(np.float32)
    t = (uu * u2 * p + uu).astype(np.float32)
    ref = np.tanh(uu.astype(np.float64))
    return float(np.max(np.abs(t.astype(np.float64) - ref) / ref))


if __name__ == "__main__":
    coeffs = fit()
    for i, c in enumerate(coeffs):
        print(f"c{i + 1} (u^{2 * i + 3}) = {float(np.float32(c))!r}")
    print("max relative error (fp32 Horner):", max_rel_error_fp32(coeffs))
