"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises ``AssertionError``
when the oracle disagrees with what the pages and the mathematics fix:
hand-derived closed forms (``tests/golden/closed_forms.json``), invariants
(sum of probabilities, Gibbs inequality, KL(p, p) = 0, shift invariance,
linearity of the top-k gradient), special cases that reduce to a library
routine (torch fp64 ``log_softmax`` / ``tanh`` / ``kl_div`` and autograd), brute
force on tiny rows and central finite differences.

The same functions run twice: once against the real oracle (every pin must
pass) and once against deliberately broken copies of it (every copy must fail
at least one pin), so a plausible slip in the oracle cannot go unnoticed.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")

_NS = {"log": math.log, "atanh": math.atanh, "inf": math.inf, "nan": math.nan,
       "exp": math.exp, "sqrt": math.sqrt}


def ev(e):
    """Evaluate one golden expression (numbers pass through)."""
    if isinstance(e, (int, float)):
        return float(e)
    return float(eval(e, {"__builtins__": {}}, _NS))  # noqa: S307 - fixture file in this repo


def ev_arr(a):
    return np.array([[ev(v) for v in row] for row in a]) if isinstance(a[0], list) else \
        np.array([ev(v) for v in a])


def golden_cases(op=None):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    return [c for c in cases if op is None or c["op"] == op]


def close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    same_class = (np.isnan(a) == np.isnan(b)) & (np.isposinf(a) == np.isposinf(b)) & \
        (np.isneginf(a) == np.isneginf(b))
    assert same_class.all(), f"{what}: non-finite placement differs\n{a}\n{b}"
    fin = np.isfinite(a)
    err = np.abs(a[fin] - b[fin])
    tol = atol + rtol * np.abs(b[fin])
    assert (err <= tol).all(), f"{what}: max err {err.max() if err.size else 0} \n{a}\n{b}"


def rng(seed=0):
    return np.random.default_rng(seed)


def _cap_t(x, cap):
    return cap * torch.tanh(x / cap) if cap else x


# ------------------------------------------------------------------ softcap

def pin_softcap_golden(orc):
    for c in golden_cases("softcap"):
        for case in c["cases"]:
            x = np.array([ev(case["x"])])
            y = orc.softcap_fwd(x, case["cap"])
            s = orc.softcap_bwd(x, np.ones(1), case["cap"])
            close(y, [ev(case["y"])], 1e-14, 1e-14, "softcap y")
            close(s, [ev(case["slope"])], 1e-14, 1e-14, "softcap slope")


def pin_softcap_torch_tanh(orc):
    r = rng(1)
    for cap in (20.0, 30.0):
        x = r.normal(0, cap / 2, 4096) * r.choice([0.01, 1, 5], 4096)
        y = orc.softcap_fwd(x, cap)
        ref = (cap * torch.tanh(torch.from_numpy(x) / cap)).numpy()
        close(y, ref, 1e-14, 1e-14, "softcap vs torch.tanh")


def pin_softcap_central_difference(orc):
    r = rng(2)
    for cap in (20.0, 30.0):
        x = r.normal(0, cap, 512)
        h = 1e-5 * cap
        fd = (orc.softcap_fwd(x + h, cap) - orc.softcap_fwd(x - h, cap)) / (2 * h)
        gy = r.normal(0, 1, 512)
        gx = orc.softcap_bwd(x, gy, cap)
        close(gx, gy * fd, 1e-7, 1e-9, "softcap grad vs central difference")


def pin_softcap_cap_cancels(orc):
    # At fixed u = x/c the slope is 1 - tanh^2(u) for every cap: the outer c and
    # the inner 1/c multiply to one.
    u = np.linspace(-6, 6, 97)
    s20 = orc.softcap_bwd(20.0 * u, np.ones_like(u), 20.0)
    s30 = orc.softcap_bwd(30.0 * u, np.ones_like(u), 30.0)
    close(s20, s30, 1e-13, 1e-15, "slope independent of cap")
    close(s20, 1 - np.tanh(u) ** 2, 1e-12, 1e-15, "slope = 1 - tanh^2")


def pin_softcap_saturation(orc):
    for cap in (20.0, 30.0):
        x = np.array([20 * cap, -20 * cap, 1000.0 + 25 * cap, -np.inf, np.inf])
        y = orc.softcap_fwd(x, cap)
        assert (y == np.array([cap, -cap, cap, -cap, cap])).all(), y
        s = orc.softcap_bwd(x, np.ones_like(x), cap)
        assert (np.abs(s) < 1e-16).all() and (s[3:] == 0).all(), s


# ----------------------------------------------------------------- logprobs

def pin_logp_golden(orc):
    for c in golden_cases("logp"):
        x = ev_arr(c["x"])
        t = np.array(c["targets"], dtype=np.int64)
        out = orc.logp_fwd(x, t, c["cap"])
        close(out, ev_arr(c["out"]), 1e-14, 1e-15, c["name"] + " out")
        gx = orc.logp_bwd(x, t, np.array(c["grad"]), c["cap"])
        close(gx, ev_arr(c["grad_x"]), 1e-14, 1e-15, c["name"] + " grad")


def _masked_rows(r, N, V, scale=3.0):
    x = r.normal(0, scale, (N, V))
    mask = r.random((N, V)) < 0.2
    x[mask] = -np.inf
    x[np.arange(N), r.integers(0, V, N)] = r.normal(0, scale, N)   # keep rows non-empty
    return x


def pin_logp_torch_log_softmax(orc):
    r = rng(3)
    for cap in (0.0, 20.0):
        x = _masked_rows(r, 16, 257)
        t = np.tile(np.arange(257), (16, 1))
        out = orc.logp_fwd(x, t, cap)
        ref = torch.log_softmax(_cap_t(torch.from_numpy(x), cap), dim=-1).numpy()
        if cap:
            close(out, ref, 1e-12, 1e-12, "logp vs torch.log_softmax (capped)")
        else:
            close(out, ref, 1e-12, 1e-12, "logp vs torch.log_softmax")


def pin_logp_probabilities_sum_to_one(orc):
    r = rng(4)
    for V in (1, 2, 7, 1031):
        x = _masked_rows(r, 5, V, 4.0) if V > 2 else r.normal(0, 4, (5, V))
        t = np.tile(np.arange(V), (5, 1))
        p = np.exp(orc.logp_fwd(x, t))
        s = np.array([math.fsum(row) for row in p])
        assert np.all(np.abs(s - 1) <= V * 2.0 ** -50), s


def pin_logp_tiny_vocab_closed_form(orc):
    r = rng(5)
    x1 = r.normal(0, 3, (6, 1))
    assert (orc.logp_fwd(x1, np.zeros((6, 1), np.int64)) == 0).all()
    assert (orc.logp_bwd(x1, np.zeros((6, 1), np.int64), r.normal(0, 1, (6, 1))) == 0).all()
    x2 = r.normal(0, 3, (8, 2))
    t = r.integers(0, 2, 8)
    other = x2[np.arange(8), 1 - t]
    mine = x2[np.arange(8), t]
    close(orc.logp_fwd(x2, t), -np.log1p(np.exp(other - mine)), 1e-13, 1e-15, "V=2 logp")


def pin_logp_shift_invariance(orc):
    r = rng(6)
    x = r.normal(0, 3, (4, 300))
    t = r.integers(0, 300, 4)
    g = r.normal(0, 1, 4)
    close(orc.logp_fwd(x + 1000.0, t), orc.logp_fwd(x, t), 1e-10, 1e-10, "logp +1000")
    close(orc.logp_bwd(x + 1000.0, t, g), orc.logp_bwd(x, t, g), 1e-9, 1e-12, "grad +1000")


def pin_logp_gradient_sums_to_zero(orc):
    r = rng(7)
    x = r.normal(0, 3, (8, 513))
    t = r.integers(0, 513, 8)
    gx = orc.logp_bwd(x, t, r.normal(0, 1, 8))
    assert np.all(np.abs(gx.sum(axis=1)) < 1e-12), gx.sum(axis=1)


def pin_logp_topk_linearity(orc):
    r = rng(8)
    V, k = 50, 6
    x = r.normal(0, 2, (3, V))
    t = r.integers(0, V, (3, k))
    t[0, 1] = t[0, 0]           # duplicate
    t[1, 2] = -100              # ignored
    g = r.normal(0, 1, (3, k))
    whole = orc.logp_bwd(x, t, g, 20.0)
    parts = np.zeros_like(whole)
    for j in range(k):
        parts += orc.logp_bwd(x, t[:, j:j + 1], g[:, j:j + 1], 20.0)
    close(whole, parts, 1e-12, 1e-14, "top-k grad = sum of single-target grads")


def _fd_check(f, x, grad, h=1e-6, what=""):
    """Directional central difference of the scalar f at x along random dirs.

    Truncation error is O(h^2) and rounding error O(1e-16 |f| / h), both far
    below the 1e-6 bound; a dropped or mis-signed term moves the result by O(1).
    """
    r = rng(99)
    for _ in range(4):
        d = r.normal(0, 1, x.shape)
        fd = (f(x + h * d) - f(x - h * d)) / (2 * h)
        an = float((grad * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{what}: fd {fd} vs analytic {an}"


def pin_logp_finite_difference(orc):
    r = rng(9)
    for cap in (0.0, 30.0):
        x = r.normal(0, 4, (3, 40))
        t = r.integers(0, 40, (3, 3))
        g = r.normal(0, 1, (3, 3))
        f = lambda z: float((orc.logp_fwd(z, t, cap) * g).sum())  # noqa: E731
        _fd_check(f, x, orc.logp_bwd(x, t, g, cap), what=f"logp fd cap={cap}")


def pin_logp_torch_autograd(orc):
    r = rng(10)
    for cap in (0.0, 20.0):
        x = r.normal(0, 5, (6, 77))
        t = r.integers(0, 77, (6, 4))
        g = r.normal(0, 1, (6, 4))
        xt = torch.from_numpy(x).requires_grad_(True)
        lp = torch.log_softmax(_cap_t(xt, cap), dim=-1).gather(1, torch.from_numpy(t))
        (lp * torch.from_numpy(g)).sum().backward()
        close(orc.logp_bwd(x, t, g, cap), xt.grad.numpy(), 1e-11, 1e-13, "logp vs autograd")


def pin_logp_ignored_targets(orc):
    r = rng(11)
    V = 64
    x = r.normal(0, 3, (5, V))
    t = np.array([[3, -100], [V, 5], [V + 7, -1], [0, V - 1], [-100, -100]])
    g = r.normal(0, 1, (5, 2))
    out = orc.logp_fwd(x, t)
    assert out[0, 1] == 0 and out[1, 0] == 0 and (out[2] == 0).all() and (out[4] == 0).all()
    gx = orc.logp_bwd(x, t, g)
    assert (gx[2] == 0).all() and (gx[4] == 0).all()
    # a row with one ignored slot equals the row with that slot dropped
    close(gx[0], orc.logp_bwd(x[:1], t[:1, :1], g[:1, :1])[0], 0, 0, "ignored slot dropped")
    close(gx[1], orc.logp_bwd(x[1:2], t[1:2, 1:], g[1:2, 1:])[0], 0, 0, "ignored slot dropped")


def pin_logp_empty_and_masked(orc):
    V = 10
    x = np.zeros((3, V))
    x[0, :] = -np.inf                   # empty row
    x[1, :] = -np.inf                   # empty row, but nothing valid
    x[2, 4:] = -np.inf                  # masked tail
    t = np.array([[2], [-100], [7]])
    out = orc.logp_fwd(x, t)
    assert np.isnan(out[0, 0]) and out[1, 0] == 0 and out[2, 0] == -np.inf
    gx = orc.logp_bwd(x, t, np.array([[1.0], [1.0], [2.0]]))
    assert np.isnan(gx[0]).all() and (gx[1] == 0).all()
    # masked target column: only its one-hot term; other masked columns exactly 0
    assert gx[2, 7] == 2.0 and (gx[2, 4:7] == 0).all() and (gx[2, 8:] == 0).all()
    close(gx[2, :4], -2.0 * np.full(4, 0.25), 1e-15, 1e-15, "masked-tail row grad")


# ------------------------------------------------------------------ entropy

def pin_entropy_golden(orc):
    for c in golden_cases("entropy"):
        x = ev_arr(c["x"])
        close(orc.entropy_fwd(x, c["cap"]), ev_arr(c["out"]), 1e-14, 1e-15, c["name"])
        gx = orc.entropy_bwd(x, np.array(c["grad"]), c["cap"])
        close(gx, ev_arr(c["grad_x"]), 1e-13, 1e-15, c["name"] + " grad")
    for c in golden_cases("entropy_uniform"):
        x = np.full((1, c["V"]), 0.75)
        # a plain running sum of V terms: relative rounding bound V * 2^-52
        close(orc.entropy_fwd(x), [ev(c["out"])], c["V"] * 2.0 ** -52, 0, c["name"])


def pin_entropy_uniform(orc):
    for V in (1, 2, 3, 1000):
        x = np.full((2, V), 7.5)
        close(orc.entropy_fwd(x), np.full(2, math.log(V)), 1e-13, 1e-15, "uniform H")
        assert np.all(np.abs(orc.entropy_bwd(x, np.ones(2))) < 1e-15)
    # saturated softcap rows: every logit caps to c, so H = log V
    x = np.full((1, 4096), 1000.0) + rng(12).normal(0, 15, (1, 4096))
    close(orc.entropy_fwd(x, 30.0), [math.log(4096)], 1e-13, 0, "saturated cap H")


def pin_entropy_bounds(orc):
    r = rng(13)
    x = _masked_rows(r, 32, 200, 6.0)
    H = orc.entropy_fwd(x)
    nf = np.isfinite(x).sum(axis=1)
    assert np.all(H >= 0) and np.all(H <= np.log(nf) + 1e-12)
    # a dominant logit drives H to 0: two-level row closed form
    # with Z = 1 + (V-1) e^-L: H = log Z + (1 - p_0) L and 1 - p_0 = (V-1) e^-L / Z
    # (the textbook log of Z = 1 + tiny loses digits as e^-L shrinks, so keep
    #  L moderate and the bound at 1e-8 relative)
    for L in (3.0, 8.0, 12.0):
        V = 100
        x2 = np.zeros((1, V))
        x2[0, 0] = L
        tail = (V - 1) * math.exp(-L)
        H2 = math.log1p(tail) + tail / (1 + tail) * L
        close(orc.entropy_fwd(x2), [H2], 1e-8, 1e-300, f"two-level entropy L={L}")


def pin_entropy_torch(orc):
    r = rng(14)
    for cap in (0.0, 30.0):
        x = _masked_rows(r, 8, 333, 8.0) if not cap else r.normal(0, 15, (8, 333))
        xt = torch.from_numpy(x).requires_grad_(True)
        lp = torch.log_softmax(_cap_t(xt, cap), dim=-1)
        H = -(torch.special.xlogy(lp.exp(), lp.exp())).sum(-1)
        close(orc.entropy_fwd(x, cap), H.detach().numpy(), 1e-11, 1e-12, "entropy vs xlogy")
        g = r.normal(0, 1, 8)
        # autograd through the finite entries only (masked logits carry p = 0)
        fin = torch.isfinite(lp)
        Hm = -(torch.where(fin, lp.exp() * torch.where(fin, lp, 0.0), 0.0)).sum(-1)
        (Hm * torch.from_numpy(g)).sum().backward()
        close(orc.entropy_bwd(x, g, cap), torch.nan_to_num(xt.grad).numpy(), 1e-10, 1e-12,
              "entropy grad vs autograd")


def pin_entropy_finite_difference(orc):
    r = rng(15)
    for cap in (0.0, 20.0):
        x = r.normal(0, 3, (3, 30))
        g = r.normal(0, 1, 3)
        f = lambda z: float((orc.entropy_fwd(z, cap) * g).sum())  # noqa: E731
        _fd_check(f, x, orc.entropy_bwd(x, g, cap), what=f"entropy fd cap={cap}")


def pin_entropy_empty_and_masked(orc):
    x = np.zeros((2, 6))
    x[0] = -np.inf
    x[1, 3:] = -np.inf
    H = orc.entropy_fwd(x)
    assert np.isnan(H[0])
    close(H[1:], [math.log(3)], 1e-14, 0, "masked-tail entropy")
    gx = orc.entropy_bwd(x, np.array([1.0, 1.0]))
    assert np.isnan(gx[0]).all() and (gx[1, 3:] == 0).all()


# ----------------------------------------------------------------------- KL

def pin_kl_golden(orc):
    for c in golden_cases("kl"):
        P, R = ev_arr(c["policy"]), ev_arr(c["ref"])
        g = np.array(c["grad"])
        close(orc.kl_fwd(P, R, 0), ev_arr(c["reverse_out"]), 1e-14, 1e-15, c["name"] + " rev")
        close(orc.kl_fwd(P, R, 1), ev_arr(c["forward_out"]), 1e-14, 1e-15, c["name"] + " fwd")
        if "reverse_grad_x" in c:
            close(orc.kl_bwd(P, R, g, 0), ev_arr(c["reverse_grad_x"]), 1e-13, 1e-15,
                  c["name"] + " rev grad")
        close(orc.kl_bwd(P, R, g, 1), ev_arr(c["forward_grad_x"]), 1e-14, 1e-15,
              c["name"] + " fwd grad")


def pin_kl_self_is_zero(orc):
    r = rng(16)
    x = _masked_rows(r, 6, 120, 3.0)
    for d in (0, 1):
        assert (orc.kl_fwd(x, x, d) == 0).all()
        assert (orc.kl_bwd(x, x, r.normal(0, 1, 6), d) == 0).all()


def pin_kl_gibbs_and_swap(orc):
    r = rng(17)
    a = r.normal(0, 3, (20, 90))
    b = a + r.normal(0, 0.5, (20, 90))
    rev = orc.kl_fwd(a, b, 0)
    fwd = orc.kl_fwd(a, b, 1)
    assert np.all(rev >= -1e-12) and np.all(fwd >= -1e-12)
    close(rev, orc.kl_fwd(b, a, 1), 1e-13, 1e-15, "KL(P||R) == forward KL with roles swapped")
    assert not np.allclose(rev, fwd), "reverse and forward KL must differ on asymmetric rows"


def pin_kl_torch_kl_div(orc):
    r = rng(18)
    for cap_p, cap_r in ((0.0, 0.0), (20.0, 30.0)):
        a = r.normal(0, 3, (10, 150))
        b = a + r.normal(0, 0.5, (10, 150))
        lpa = torch.log_softmax(_cap_t(torch.from_numpy(a), cap_p), -1)
        lpb = torch.log_softmax(_cap_t(torch.from_numpy(b), cap_r), -1)
        # kl_div(input, target, log_target) = sum target * (log target - input)
        rev = torch.nn.functional.kl_div(lpb, lpa, reduction="none", log_target=True).sum(-1)
        fwd = torch.nn.functional.kl_div(lpa, lpb, reduction="none", log_target=True).sum(-1)
        close(orc.kl_fwd(a, b, 0, cap_p, cap_r), rev.numpy(), 1e-10, 1e-13, "rev vs kl_div")
        close(orc.kl_fwd(a, b, 1, cap_p, cap_r), fwd.numpy(), 1e-10, 1e-13, "fwd vs kl_div")


def pin_kl_autograd(orc):
    r = rng(19)
    for cap_p, cap_r in ((0.0, 0.0), (30.0, 20.0)):
        a = r.normal(0, 3, (5, 64))
        b = a + r.normal(0, 0.5, (5, 64))
        g = r.normal(0, 1, 5)
        for d in (0, 1):
            at = torch.from_numpy(a).requires_grad_(True)
            lpa = torch.log_softmax(_cap_t(at, cap_p), -1)
            lpb = torch.log_softmax(_cap_t(torch.from_numpy(b), cap_r), -1)
            if d == 0:
                kl = (lpa.exp() * (lpa - lpb)).sum(-1)
            else:
                kl = (lpb.exp() * (lpb - lpa)).sum(-1)
            (kl * torch.from_numpy(g)).sum().backward()
            close(orc.kl_bwd(a, b, g, d, cap_p, cap_r), at.grad.numpy(), 1e-10, 1e-13,
                  f"KL dir={d} grad vs autograd")


def pin_kl_finite_difference(orc):
    r = rng(20)
    a = r.normal(0, 2, (3, 25))
    b = a + r.normal(0, 0.7, (3, 25))
    g = r.normal(0, 1, 3)
    for d in (0, 1):
        f = lambda z: float((orc.kl_fwd(z, b, d, 20.0, 0.0) * g).sum())  # noqa: E731
        _fd_check(f, a, orc.kl_bwd(a, b, g, d, 20.0, 0.0), what=f"KL fd dir={d}")


def pin_kl_mismatch_and_empty(orc):
    V = 8
    a = np.zeros((4, V))
    b = np.zeros((4, V))
    b[0, 6:] = -np.inf                  # reference masks what the policy supports
    a[1, 5] = -800.0                    # policy probability underflows in fp64 ...
    b[1, 5] = -np.inf                   # ... and the reference masks that column
    a[2] = -np.inf                      # empty policy row
    b[3] = -np.inf                      # empty reference row
    rev = orc.kl_fwd(a, b, 0)
    assert rev[0] == np.inf and rev[1] == np.inf and np.isnan(rev[2]) and np.isnan(rev[3])
    fwd = orc.kl_fwd(a, b, 1)
    assert np.isfinite(fwd[:2]).all() and np.isnan(fwd[2:]).all()
    g = np.array([1.0, 1.0, 1.0, 1.0])
    gf = orc.kl_bwd(a, b, g, 1)
    # forward KL: masked reference columns get exactly g * p
    close(gf[0, 6:], np.full(2, 1 / 8), 1e-15, 0, "forward KL masked-ref grad = g p")
    assert np.isfinite(gf[:2]).all() and np.isnan(gf[2:]).all()
    gr = orc.kl_bwd(a, b, g, 0)
    assert np.isnan(gr[0]).all() and np.isnan(gr[2:]).all()


def pin_kl_mismatch_limit(orc):
    """The reverse-KL gradient on a support-mismatch row as the limit of
    finite rows.  Replace the reference's -inf logits by -M: the row is then
    an ordinary one, whose gradient the autograd and finite-difference pins
    fix.  As M grows, KL grows like P_m M (P_m: the policy's mass on the
    columns the reference masks) and the gradient on the policy's support
    diverges like M (g p_v (1 - P_m) M on the masked columns, -g p_v P_m M on
    the others), so no finite value is right there, while a column off the
    policy's support (policy logit -inf) has p_v = 0 and a gradient of
    exactly 0 at every M.  The mismatch row must therefore be non-finite on
    the support (the oracle's class for it is NaN, the same marker as for
    the other rows without a defined gradient) and exactly 0 off it.  (When
    the reference masks all of the policy's support, P_m = 1, the finite
    gradients converge instead; rows here keep P_m < 1.)"""
    r = rng(25)
    V = 10
    a = r.normal(0, 1, (2, V))
    b = r.normal(0, 1, (2, V))
    a[0, 8:] = -np.inf               # off the policy's support
    b[0, [0, 1, 9]] = -np.inf        # 0, 1: the mismatch; 9: masked on both sides
    a[1, 0] = -np.inf
    b[1, [3, 4, 5]] = -np.inf
    g = np.array([1.3, -0.7])
    assert (orc.kl_fwd(a, b, 0) == np.inf).all()
    gr = orc.kl_bwd(a, b, g, 0)
    off = ~np.isfinite(a)
    masked = ~np.isfinite(b) & ~off
    pa = np.where(off, 0.0, np.exp(a - np.log(np.exp(np.where(off, -np.inf, a)).sum(-1,
                                                                                   keepdims=True))))
    pm = (pa * masked).sum(-1, keepdims=True)
    assert ((pm > 0) & (pm < 1)).all()
    rate = g[:, None] * pa * np.where(masked, 1.0 - pm, -pm)   # d grad / dM
    # Past M ~ 40 the finite row's gradient is affine in M up to terms of
    # e^-M, so its slope between two values of M is the rate itself.
    prev = None
    for M in (1e3, 1e4, 1e5, 1e6):
        gm = orc.kl_bwd(a, np.where(np.isfinite(b), b, -M), g, 0)
        assert np.isfinite(gm).all()
        assert (gm[off] == 0).all(), "a column off the support has a zero gradient at every M"
        on = gm[~off]
        if prev is not None:
            close((on - prev[1]) / (M - prev[0]), rate[~off], 1e-8, 1e-12, f"slope at M={M:g}")
            assert (np.abs(on) > np.abs(prev[1])).all(), "the support's gradient grows with M"
        prev = (M, on)
    assert (gr[off] == 0).all(), "mismatch row: zero off the policy's support"
    assert np.isnan(gr[~off]).all(), "mismatch row: non-finite (NaN) on the policy's support"


def pin_kl_masked_policy(orc):
    r = rng(21)
    a = _masked_rows(r, 4, 60, 3.0)
    b = np.where(np.isfinite(a), a + r.normal(0, 0.5, a.shape), r.normal(0, 3, a.shape))
    g = r.normal(0, 1, 4)
    gr = orc.kl_bwd(a, b, g, 0)
    assert (gr[~np.isfinite(a)] == 0).all()
    lpa = torch.log_softmax(torch.from_numpy(a), -1)
    lpb = torch.log_softmax(torch.from_numpy(b), -1)
    pa = lpa.exp()
    rev = torch.where(pa > 0, pa * (lpa - lpb), 0.0).sum(-1)
    close(orc.kl_fwd(a, b, 0), rev.numpy(), 1e-11, 1e-13, "masked-policy reverse KL")


# -- gradient with respect to the reference (not detached) -------------------

def pin_kl_ref_autograd(orc):
    r = rng(22)
    for cap_p, cap_r in ((0.0, 0.0), (30.0, 20.0)):
        a = r.normal(0, 3, (5, 64))
        b = a + r.normal(0, 0.5, (5, 64))
        g = r.normal(0, 1, 5)
        for d in (0, 1):
            bt = torch.from_numpy(b).requires_grad_(True)
            lpa = torch.log_softmax(_cap_t(torch.from_numpy(a), cap_p), -1)
            lpb = torch.log_softmax(_cap_t(bt, cap_r), -1)
            if d == 0:
                kl = (lpa.exp() * (lpa - lpb)).sum(-1)
            else:
                kl = (lpb.exp() * (lpb - lpa)).sum(-1)
            (kl * torch.from_numpy(g)).sum().backward()
            close(orc.kl_bwd_ref(a, b, g, d, cap_p, cap_r), bt.grad.numpy(), 1e-10, 1e-13,
                  f"KL dir={d} reference grad vs autograd")


def pin_kl_ref_finite_difference(orc):
    r = rng(23)
    a = r.normal(0, 2, (3, 25))
    b = a + r.normal(0, 0.7, (3, 25))
    g = r.normal(0, 1, 3)
    for d in (0, 1):
        f = lambda z: float((orc.kl_fwd(a, z, d, 0.0, 20.0) * g).sum())  # noqa: E731
        _fd_check(f, b, orc.kl_bwd_ref(a, b, g, d, 0.0, 20.0), what=f"KL ref fd dir={d}")


def pin_kl_ref_equals_policy_grad_of_swapped_roles(orc):
    # KL(P||R) is the forward KL of the pair (policy R, reference P), and the
    # other way round, so the reference gradient of one direction is the
    # policy gradient of the other with the two tensors (and caps) swapped.
    r = rng(24)
    a = _masked_rows(r, 4, 40, 3.0)
    b = np.where(np.isfinite(a), a + r.normal(0, 0.5, a.shape), -np.inf)
    g = r.normal(0, 1, 4)
    for cp, cr in ((0.0, 0.0), (20.0, 30.0)):
        for d in (0, 1):
            close(orc.kl_bwd_ref(a, b, g, d, cp, cr), orc.kl_bwd(b, a, g, 1 - d, cr, cp),
                  1e-15, 0, f"swap dir={d} caps={cp, cr}")


def pin_kl_ref_special_rows(orc):
    V = 8
    a = np.zeros((5, V))
    b = np.zeros((5, V))
    b[0, 6:] = -np.inf          # reverse mismatch: reference masks policy columns
    a[1, 5:] = -np.inf          # forward mismatch: policy masks reference columns
    a[2] = -np.inf              # empty policy row
    b[3] = -np.inf              # empty reference row
    g = np.ones(5)
    rv = orc.kl_bwd_ref(a, b, g, 0)
    # q - p: reference-masked columns get exactly -p = -1/8, the rest 1/6 - 1/8
    close(rv[0, 6:], np.full(2, -1 / 8), 1e-15, 0, "reverse KL ref grad on masked ref")
    close(rv[0, :6], np.full(6, 1 / 6 - 1 / 8), 1e-15, 1e-16, "reverse KL ref grad on support")
    close(rv[1, 5:], np.full(3, 1 / 8), 1e-15, 0, "reverse KL ref grad, policy-masked")
    assert np.isnan(rv[2:4]).all() and (rv[4] == 0).all()
    fw = orc.kl_bwd_ref(a, b, g, 1)
    assert np.isinf(orc.kl_fwd(a, b, 1)[1])
    assert np.isnan(fw[1]).all()                     # reference supports every column
    assert np.isfinite(fw[0]).all() and (fw[0, 6:] == 0).all()
    assert np.isnan(fw[2:4]).all() and (fw[4] == 0).all()
    b2 = b.copy()
    b2[1, 7] = -np.inf                               # masked reference column on a mismatch row
    fw2 = orc.kl_bwd_ref(a, b2, g, 1)
    assert fw2[1, 7] == 0 and np.isnan(fw2[1, :7]).all()


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
