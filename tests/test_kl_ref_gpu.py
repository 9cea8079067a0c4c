"""KL with a reference that is not detached, and both directions from one read.

* rlk_kl_bwd_ref against the oracle's reference gradient (every dtype, tails,
  both caps, the special rows of the policy-gradient tests plus a mismatch in
  each direction);
* rlk_kl_fwd_both: each direction's output and row record bit-identical to the
  one-direction forward, and its records drive both backward calls;
* the swapped-roles identity on the GPU: with the record's sides exchanged,
  the reference gradient of KL(P||R) is bit for bit the policy gradient of
  the forward KL of the pair (R, P);
* strided views and the autograd function with ``detach_ref=False``.
"""

import numpy as np
import pytest
import torch

from tests.parity import assert_grad, assert_out, to64
from tests.test_parity_gpu import DT_IDS, DTYPES, gen, kl_pair
from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8).cpu()


def pair(N, V, dtype, seed, caps):
    cp, cr = caps
    a, b = kl_pair(N, V, torch.float32, seed, mismatch_rows=(1,) if not cr else (),
                   empty_rows=(3,) if not (cp or cr) else (),
                   both_masked_rows=(5,) if not (cp or cr) else (),
                   underflow_row=7 if not (cp or cr) else None)
    if not cp and V >= 2:
        a[8, V // 2:] = float("-inf")     # policy masks what the reference supports
    if not cr:
        b[9] = float("-inf")              # empty reference only
    return a.to(dtype), b.to(dtype)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("V", [2, 7, 1031, 4097, 32000])
@pytest.mark.parametrize("direction", [0, 1], ids=["rev", "fwd"])
@pytest.mark.parametrize("caps", [(0.0, 0.0), (30.0, 20.0), (0.0, 25.0), (50.0, 20.0)],
                         ids=["nocap", "cap", "refcap", "online_fixed"])
def test_kl_reference_gradient(dev, orc, dtype, V, direction, caps):
    N = 12
    cp, cr = caps
    a, b = pair(N, V, dtype, V + 31, caps)
    g = torch.randn(N, generator=gen(V + 32))
    ad, bd = a.to(dev), b.to(dev)
    D, stats = rlk.kl_fwd(ad, bd, direction, cp, cr)
    gr = rlk.kl_bwd_ref(ad, bd, g.to(dev), stats, direction, cp, cr)
    torch.cuda.synchronize()
    a64, b64 = to64(a), to64(b)
    assert_out(D, orc.kl_fwd(a64, b64, direction, cp, cr), dtype, "kl")
    ez = None
    if direction == 1 and not cr:
        # forward KL: the reference's masked columns get exactly 0
        ez = np.isneginf(b64) & ~np.isneginf(b64).all(1, keepdims=True)
        ez &= ~np.isneginf(a64).all(1, keepdims=True)
    assert_grad(gr, orc.kl_bwd_ref(a64, b64, to64(g), direction, cp, cr), "kl ref grad",
                exact_zero=ez)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("V", [7, 4099, 75968])
@pytest.mark.parametrize("caps", [(0.0, 0.0), (30.0, 20.0), (20.0, 50.0)],
                         ids=["nocap", "cap", "fixed_online"])
def test_both_directions_forward_is_bitwise_single(dev, orc, dtype, V, caps):
    N = 12
    cp, cr = caps
    a, b = pair(N, V, dtype, V + 41, caps)
    ad, bd = a.to(dev), b.to(dev)
    rv, srv, fw, sfw = rlk.kl_fwd_both(ad, bd, cp, cr)
    rv1, srv1 = rlk.kl_fwd(ad, bd, 0, cp, cr)
    fw1, sfw1 = rlk.kl_fwd(ad, bd, 1, cp, cr)
    torch.cuda.synchronize()
    for x, y, what in ((rv, rv1, "reverse"), (srv, srv1, "reverse record"),
                       (fw, fw1, "forward"), (sfw, sfw1, "forward record")):
        assert torch.equal(_bits(x), _bits(y)), what
    a64, b64 = to64(a), to64(b)
    assert_out(rv, orc.kl_fwd(a64, b64, 0, cp, cr), dtype, "reverse vs oracle")
    assert_out(fw, orc.kl_fwd(a64, b64, 1, cp, cr), dtype, "forward vs oracle")
    # the records drive both backward calls of their direction
    g = torch.randn(N, generator=gen(V + 42)).to(dev)
    for d, st in ((0, srv), (1, sfw)):
        gp = rlk.kl_bwd(ad, bd, g, st, d, cp, cr)
        gr = rlk.kl_bwd_ref(ad, bd, g, st, d, cp, cr)
        torch.cuda.synchronize()
        assert_grad(gp, orc.kl_bwd(a64, b64, to64(g), d, cp, cr), f"policy grad d={d}")
        assert_grad(gr, orc.kl_bwd_ref(a64, b64, to64(g), d, cp, cr), f"ref grad d={d}")


def swap_record(st):
    """The row record with its policy (a) and reference (b) sides exchanged."""
    s = st.view(torch.float32).reshape(-1, 8).clone()
    s[:, [0, 1, 2, 3]] = s[:, [2, 3, 0, 1]]
    f = s[:, 5].contiguous().view(torch.int32)
    f = (f & 4) | ((f & 1) << 1) | ((f & 2) >> 1)   # empty-a <-> empty-b, mismatch kept
    s[:, 5] = f.view(torch.float32)
    return s.view(torch.uint8).reshape(st.shape)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("caps", [(0.0, 0.0), (30.0, 20.0), (50.0, 20.0)],
                         ids=["nocap", "cap", "online_fixed"])
def test_reference_gradient_is_policy_gradient_of_swapped_pair(dev, dtype, caps):
    # KL(P||R) is the forward KL of the pair (policy R, reference P): with the
    # record's sides exchanged, the policy gradient of the swapped pair is the
    # reference gradient bit for bit.  The swapped forward itself agrees to
    # rounding (its online rescales run in the other order).
    N, V = 12, 5003
    cp, cr = caps
    a, b = pair(N, V, dtype, 51, caps)
    ad, bd = a.to(dev), b.to(dev)
    g = torch.randn(N, generator=gen(52)).to(dev)
    for d in (0, 1):
        D, st = rlk.kl_fwd(ad, bd, d, cp, cr)
        Ds, _ = rlk.kl_fwd(bd, ad, 1 - d, cr, cp)
        gr = rlk.kl_bwd_ref(ad, bd, g, st, d, cp, cr)
        gs = rlk.kl_bwd(bd, ad, g, swap_record(st), 1 - d, cr, cp)
        torch.cuda.synchronize()
        torch.testing.assert_close(D, Ds, rtol=4e-6, atol=1e-7, equal_nan=True)
        assert torch.equal(_bits(gr), _bits(gs)), f"gradient, d={d}"


def test_strided_both_and_reference_gradient(dev, orc):
    B, T, V = 3, 5, 3001
    full_a = torch.randn(B, T + 1, V, generator=gen(61)) * 3
    full_b = full_a + torch.randn(B, T + 1, V, generator=gen(62)) * 0.5
    full_a[:, -1] = float("nan")        # outside the view
    full_b[:, -1] = float("nan")
    a, b = full_a.to(torch.bfloat16).to(dev), full_b.to(torch.bfloat16).to(dev)
    av, bv = a[:, :-1], b[:, :-1]
    rv, srv, fw, sfw = rlk.kl_fwd_both(av, bv)
    g = torch.randn(B, T, generator=gen(63)).to(dev)
    gbuf = torch.full((B, T + 1, V), float("nan"), dtype=torch.bfloat16, device=dev)
    rlk.kl_bwd_ref(av, bv, g, sfw, 1, out=gbuf[:, :-1])
    torch.cuda.synchronize()
    a64 = to64(av.reshape(-1, V))
    b64 = to64(bv.reshape(-1, V))
    assert_out(rv.reshape(-1), orc.kl_fwd(a64, b64, 0), torch.bfloat16, "strided reverse")
    assert_out(fw.reshape(-1), orc.kl_fwd(a64, b64, 1), torch.bfloat16, "strided forward")
    assert_grad(gbuf[:, :-1].reshape(-1, V), orc.kl_bwd_ref(a64, b64, to64(g).reshape(-1), 1),
                "strided ref grad")
    assert torch.isnan(gbuf[:, -1].float()).all()   # nothing written outside the view


@pytest.mark.parametrize("direction", [0, 1], ids=["rev", "fwd"])
def test_autograd_reaches_both_inputs(dev, orc, direction):
    V = 2000
    a = torch.randn(3, V, generator=gen(72)) * 3
    b = a + torch.randn(3, V, generator=gen(73)) * 0.5
    ad = a.to(dev).requires_grad_(True)
    bd = b.to(dev).requires_grad_(True)
    w = torch.randn(3, generator=gen(74))
    kl = rlk.kl_divergence(ad, bd, direction, detach_ref=False)
    (kl * w.to(dev)).sum().backward()
    a64, b64 = to64(a), to64(b)
    assert_grad(ad.grad, orc.kl_bwd(a64, b64, to64(w), direction), "policy grad")
    assert_grad(bd.grad, orc.kl_bwd_ref(a64, b64, to64(w), direction), "ref grad")
    # detached reference (the default) gets no gradient
    bd2 = b.to(dev).requires_grad_(True)
    rlk.kl_divergence(ad, bd2, direction).sum().backward()
    assert bd2.grad is None
