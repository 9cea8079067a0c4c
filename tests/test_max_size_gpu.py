"""The largest accepted row, V = 2^31 - 1, against closed forms.

A row this wide holds 2^31 - 1 logits (4 GiB in bf16), beyond what the fp64
oracle can hold in memory, so the rows are built so that every output has a
closed form (no oracle involved):

* row 0: every logit 0 except the target column, -4.  With Z = V - 1 + e^-4,
  logp(target) = -4 - log Z, p(other) = 1 / Z, the gradient of logp with
  upstream g is g (1 - e^-4 / Z) at the target and -g / Z elsewhere, and the
  entropy is log Z + 4 e^-4 / Z;
* row 1: every logit -inf except the last three columns (1, 2, 3): the bulk is
  masked (probability 0, gradient exactly 0 in every head) and the tail sits
  at element offsets near 2^31 of the row and 2^32 of the tensor;
* KL of the tensor against itself is exactly 0, with an exactly zero gradient.

Sampled columns (both ends, the target, a seeded random set) are compared;
the per-row sums go through 64-bit offsets, int64 chunk indices and the
vectorised tail.
"""

import math

import numpy as np
import pytest
import torch

from tests.parity import assert_grad, assert_out
from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu

V = 2**31 - 1


@pytest.fixture(scope="module")
def rows(dev):
    x = torch.zeros(2, V, dtype=torch.bfloat16, device=dev)
    t0 = 1_234_567_891
    x[0, t0] = -4.0
    x[1, : V - 3] = float("-inf")
    x[1, V - 3:] = torch.tensor([1.0, 2.0, 3.0], dtype=torch.bfloat16, device=dev)
    t = torch.tensor([[t0], [V - 1]], dtype=torch.int64, device=dev)
    yield x, t, t0
    del x
    torch.cuda.empty_cache()


def _cols(t0):
    g = np.random.default_rng(3)
    c = np.concatenate([np.arange(0, 1000), np.arange(V - 1000, V), [t0 - 1, t0, t0 + 1],
                        g.integers(0, V, 3000)])
    return torch.from_numpy(np.unique(c))


def test_logp_at_max_width(dev, rows):
    x, t, t0 = rows
    g = torch.tensor([[1.5], [-0.75]], device=dev)
    lp, st = rlk.logp_fwd(x, t)
    gx = rlk.logp_bwd(x, t, g, st)
    torch.cuda.synchronize()
    Z = (V - 1) + math.exp(-4.0)
    tail = math.log(math.e + math.e**2 + math.e**3)
    assert_out(lp, np.array([[-4.0 - math.log(Z)], [3.0 - tail]]), torch.bfloat16, "logp")
    cols = _cols(t0)
    got0 = gx[0, cols.to(dev)]
    want0 = np.full(cols.numel(), -1.5 / Z)
    want0[cols.numpy() == t0] = 1.5 * (1.0 - math.exp(-4.0) / Z)
    assert_grad(got0, want0, "row 0 grad")
    # the background values (~7e-10) are far below the absolute bound: also
    # hold them to one bf16 rounding
    rel = np.abs(got0.double().cpu().numpy() - want0) / np.abs(want0)
    assert rel.max() <= 2.0**-8, f"row 0 grad relative error {rel.max():.3g}"
    got1 = gx[1, cols.to(dev)]
    p_tail = np.exp(np.array([1.0, 2.0, 3.0]) - tail)
    want1 = np.zeros(cols.numel())
    for j, p in enumerate(p_tail):
        want1[cols.numpy() == V - 3 + j] = -0.75 * ((1.0 if j == 2 else 0.0) - p)
    assert_grad(got1, want1, "row 1 grad", exact_zero=cols.numpy() < V - 3)


def test_entropy_at_max_width(dev, rows):
    x, _, t0 = rows
    g = torch.tensor([2.0, 1.0], device=dev)
    H, st = rlk.entropy_fwd(x)
    gx = rlk.entropy_bwd(x, g, st)
    torch.cuda.synchronize()
    Z = (V - 1) + math.exp(-4.0)
    H0 = math.log(Z) + 4.0 * math.exp(-4.0) / Z
    lt = np.array([1.0, 2.0, 3.0])
    lp1 = lt - math.log(np.exp(lt).sum())
    H1 = float(-(np.exp(lp1) * lp1).sum())
    assert_out(H, np.array([H0, H1]), torch.bfloat16, "entropy")
    cols = _cols(t0)
    # row 0: d H / d x_v = -p_v (log p_v + H); p_v = 1/Z off the target
    want0 = np.full(cols.numel(), -2.0 * (1.0 / Z) * (-math.log(Z) + H0))
    pt = math.exp(-4.0) / Z
    want0[cols.numpy() == t0] = -2.0 * pt * (math.log(pt) + H0)
    # (off the target log p + H cancels to 4e^-4/Z ~ 3e-11, far below what
    # fp32 resolves next to log Z ~ 21.5: only the absolute bound applies)
    assert_grad(gx[0, cols.to(dev)], want0, "entropy row 0 grad")
    want1 = np.zeros(cols.numel())
    for j in range(3):
        want1[cols.numpy() == V - 3 + j] = -1.0 * math.exp(lp1[j]) * (lp1[j] + H1)
    assert_grad(gx[1, cols.to(dev)], want1, "entropy row 1 grad",
                exact_zero=cols.numpy() < V - 3)


def test_kl_self_at_max_width(dev, rows):
    x, _, t0 = rows
    for d in (0, 1):
        D, st = rlk.kl_fwd(x, x, d)
        gx = rlk.kl_bwd(x, x, torch.ones(2, device=dev), st, d)
        torch.cuda.synchronize()
        assert (D == 0).all(), f"KL(x, x) = {D.tolist()} (direction {d})"
        cols = _cols(t0).to(dev)
        assert (gx[0, cols] == 0).all() and (gx[1, cols] == 0).all()
        del gx
