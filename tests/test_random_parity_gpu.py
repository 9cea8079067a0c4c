"""Seeded random sweep of the HIP path against the fp64 oracle.

Each case draws, from its own seed, a head (logprobs with k between 1 and
300, entropy, KL in either direction with the reference gradient), a dtype,
a shape (V from 1 to 40000, ragged), the caps of both tensors (off, the
fixed-reference form, the running-max form, both sides of the threshold
between them), a memory layout (contiguous, padded row stride with NaN in the
padding, misaligned base pointer, [B, T, V] view with a poisoned position) and
special rows (masked columns, an all -inf row, a +1000 offset row, ignored,
out-of-range and duplicate targets).  The structured parity tests pin each of
these one at a time; the sweep checks their combinations, and so every
backward kernel (one-shot pieces for k <= 4, wide pieces for k <= 256, the
row kernel beyond) under every layout and cap form.
"""

import numpy as np
import pytest
import torch

from tests.parity import assert_grad, assert_out, to64
from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu

N_CASES = 96
DTYPES = [torch.float32, torch.bfloat16, torch.float16]
CAPS = [0.0, 0.0, 20.0, 41.5, 41.7, 60.0]
KS = [1, 2, 4, 5, 17, 64, 256, 257, 300]


def draw(i):
    r = np.random.default_rng(9000 + i)
    c = {
        "head": ["logp", "logp", "entropy", "kl0", "kl1"][int(r.integers(5))],
        "dtype": DTYPES[int(r.integers(3))],
        "V": (int(r.choice([1, 2, 3, 7, 8])) if r.random() < 0.1
              else int(np.exp(r.uniform(np.log(8.0), np.log(40000.0))))),
        "N": int(r.integers(1, 25)),
        "cap": CAPS[int(r.integers(len(CAPS)))],
        "cap_ref": CAPS[int(r.integers(len(CAPS)))],
        "layout": ["contig", "padded", "misaligned", "view3"][int(r.integers(4))],
        "k": KS[int(r.integers(len(KS)))],
        "seed": 9000 + i,
    }
    if c["layout"] == "view3" and c["N"] % 2:
        c["N"] += 1
    return c


def make_logits(c, g):
    N, V, cap = c["N"], c["V"], c["cap"]
    x = torch.randn(N, V, generator=g) * (cap / 2 if cap else 3.0)
    if N > 2:
        x[N // 2] += 1000.0                       # offset row
    if not cap and V > 2:
        m = torch.rand(N, V, generator=g) < 0.1   # masked columns, one kept per row
        m[torch.arange(N), torch.randint(0, V, (N,), generator=g)] = False
        x[m] = float("-inf")
        if N > 3:
            x[N - 1] = float("-inf")              # an all -inf row
    return x


def place(x, layout, dev):
    """x (CPU, final dtype) laid out on the device as the case asks."""
    N, V = x.shape
    if layout == "padded":
        buf = torch.full((N, V + 5), float("nan"), dtype=x.dtype, device=dev)
        buf[:, :V] = x.to(dev)
        return buf[:, :V]
    if layout == "misaligned":
        buf = torch.empty(N * V + 1, dtype=x.dtype, device=dev)
        v = buf[1:].view(N, V)
        v.copy_(x.to(dev))
        return v
    if layout == "view3":
        B, T = 2, N // 2
        buf = torch.full((B, T + 1, V), float("nan"), dtype=x.dtype, device=dev)
        buf[:, :T] = x.view(B, T, V).to(dev)
        return buf[:, :T]
    return x.to(dev)


def rows2d(t):
    return t.reshape(-1, t.shape[-1])


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(dev, orc, i):
    c = draw(i)
    g = torch.Generator().manual_seed(c["seed"])
    N, V, dt, head = c["N"], c["V"], c["dtype"], c["head"]
    print(f"case {i}: {c}", flush=True)
    x = make_logits(c, g).to(dt)
    x64 = to64(x)
    xd = place(x, c["layout"], dev)
    three = xd.dim() == 3

    if head == "logp":
        k = c["k"]
        t = torch.randint(0, V, (N, k), generator=g)
        if k > 1:
            t[:, k // 2] = t[:, 0]                # duplicates
        t[0, 0] = -100
        if N > 1:
            t[1, -1] = V + 7                      # out of range
        if N > 4:
            t[4] = -100                           # no valid slot
        gt = torch.randn(N, k, generator=g)
        ts = t.view(2, N // 2, k) if three else t
        gs = gt.view(2, N // 2, k) if three else gt
        out, st = rlk.logp_fwd(xd, ts.to(dev), c["cap"])
        gx = rlk.logp_bwd(xd, ts.to(dev), gs.to(dev), st, c["cap"])
        torch.cuda.synchronize()
        ign = ((t < 0) | (t >= V)).numpy()
        assert_out(rows2d(out), orc.logp_fwd(x64, t.numpy(), c["cap"]), dt, "logp",
                   exact_zero=ign)
        assert_grad(rows2d(gx), orc.logp_bwd(x64, t.numpy(), to64(gt), c["cap"]), "logp grad",
                    exact_zero=np.repeat(ign.all(1)[:, None], V, 1))
    elif head == "entropy":
        gr = torch.randn(N, generator=g)
        H, st = rlk.entropy_fwd(xd, c["cap"])
        gx = rlk.entropy_bwd(xd, gr.view(2, N // 2).to(dev) if three else gr.to(dev), st,
                             c["cap"])
        torch.cuda.synchronize()
        assert_out(H.reshape(-1), orc.entropy_fwd(x64, c["cap"]), dt, "entropy")
        masked = (np.isneginf(x64) & ~np.isneginf(x64).all(1, keepdims=True)
                  if not c["cap"] else None)
        assert_grad(rows2d(gx), orc.entropy_bwd(x64, to64(gr), c["cap"]), "entropy grad",
                    exact_zero=masked)
    else:
        d = int(head[2])
        cp, cr = c["cap"], c["cap_ref"]
        y = (x.double() + torch.randn(N, V, generator=g) * 0.5).to(dt)
        if not cr and N > 1 and V > 3:
            y[N - 2, V - V // 4:] = float("-inf")  # reference-only mask (mismatch)
        y64 = to64(y)
        yd = place(y, c["layout"], dev)
        gr = torch.randn(N, generator=g)
        grd = gr.view(2, N // 2).to(dev) if three else gr.to(dev)
        D, st = rlk.kl_fwd(xd, yd, d, cp, cr)
        gx = rlk.kl_bwd(xd, yd, grd, st, d, cp, cr)
        gy = rlk.kl_bwd_ref(xd, yd, grd, st, d, cp, cr)
        torch.cuda.synchronize()
        assert_out(D.reshape(-1), orc.kl_fwd(x64, y64, d, cp, cr), dt, f"kl {d}")
        assert_grad(rows2d(gx), orc.kl_bwd(x64, y64, to64(gr), d, cp, cr), f"kl {d} grad")
        assert_grad(rows2d(gy), orc.kl_bwd_ref(x64, y64, to64(gr), d, cp, cr),
                    f"kl {d} reference grad")
