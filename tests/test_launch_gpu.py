"""Launch-level behaviour of the HIP path.

* more rows than one backward launch covers (the piece grid's second
  dimension holds at most 65536 rows, so the rows are launched in slices);
* HIP graph capture: the entry points allocate nothing and record no memset,
  so a forward + backward step can be captured once and replayed; every replay
  (with eager work and synchronisations in between) must equal the eager
  result bit for bit.
"""

import numpy as np
import pytest
import torch

from tests.parity import assert_grad, assert_out, to64
from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu


def _gen(seed):
    return torch.Generator().manual_seed(seed)


@pytest.mark.parametrize("head", ["logp", "logp_k9", "entropy", "kl"])
def test_more_rows_than_one_launch(dev, orc, head):
    N, V = 70_001, 37
    x = (torch.randn(N, V, generator=_gen(1)) * 3).to(torch.bfloat16)
    g = torch.randn(N, generator=_gen(2))
    xd, gd = x.to(dev), g.to(dev)
    x64 = to64(x)
    if head.startswith("logp"):
        k = 9 if head == "logp_k9" else 1   # wide top-k pieces / one-shot pieces
        t = torch.randint(0, V, (N, k), generator=_gen(3))
        t[::97] = -100
        gt = torch.randn(N, k, generator=_gen(5))
        out, st = rlk.logp_fwd(xd, t.to(dev))
        gx = rlk.logp_bwd(xd, t.to(dev), gt.to(dev), st)
        ref_out = orc.logp_fwd(x64, t.numpy())
        ref_gx = orc.logp_bwd(x64, t.numpy(), to64(gt))
    elif head == "entropy":
        out, st = rlk.entropy_fwd(xd)
        gx = rlk.entropy_bwd(xd, gd, st)
        ref_out, ref_gx = orc.entropy_fwd(x64), orc.entropy_bwd(x64, to64(g))
    else:
        r = (x.float() + torch.randn(N, V, generator=_gen(4)) * 0.5).to(torch.bfloat16)
        rd, r64 = r.to(dev), to64(r)
        out, st = rlk.kl_fwd(xd, rd)
        gx = rlk.kl_bwd(xd, rd, gd, st)
        ref_out, ref_gx = orc.kl_fwd(x64, r64), orc.kl_bwd(x64, r64, to64(g))
    torch.cuda.synchronize()
    assert_out(out, ref_out, torch.bfloat16, f"{head} out")
    assert_grad(gx, ref_gx, f"{head} grad")


@pytest.mark.parametrize("cap", [0.0, 30.0, 50.0])
def test_graph_capture_replays_equal_eager(dev, cap):
    N, V, k = 96, 50_000, 3
    x = (torch.randn(N, V, generator=_gen(5)) * 4).to(torch.bfloat16).to(dev)
    ref = (x.float() + 0.3).to(torch.bfloat16)
    t = torch.randint(0, V, (N, k), generator=_gen(6)).to(dev)
    g = torch.randn(N, k, generator=_gen(7)).to(dev)
    gr = torch.randn(N, generator=_gen(8)).to(dev)
    lp = torch.empty(N, k, device=dev)
    h = torch.empty(N, device=dev)
    d = torch.empty(N, device=dev)
    st = [rlk.new_stats(hd, N, V, dev) for hd in (0, 1, 2)]
    gx = [torch.empty_like(x) for _ in range(3)]

    def step():
        rlk.rlk_logp_fwd(x, t, cap, lp, st[0])
        rlk.rlk_logp_bwd(x, t, cap, st[0], g, gx[0])
        rlk.rlk_entropy_fwd(x, cap, h, st[1])
        rlk.rlk_entropy_bwd(x, cap, st[1], gr, gx[1])
        rlk.rlk_kl_fwd(x, ref, 0, cap, 0.0, d, st[2])
        rlk.rlk_kl_bwd(x, ref, 0, cap, 0.0, st[2], gr, gx[2])

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    want = [a.clone() for a in (lp, h, d, *gx)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for a in (lp, h, d, *gx):       # eager work between replays
            a.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, w) in enumerate(zip((lp, h, d, *gx), want)):
            av = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
            wv = w.contiguous().view(torch.int16 if w.element_size() == 2 else torch.int32)
            assert torch.equal(av, wv), f"replay {rep}: output {i} differs from eager"


def test_prepared_calls_repeat_the_direct_call(dev):
    # prepare() marshals once; every call of the result is the same C call
    N, V, k = 5, 3000, 2
    x = (torch.randn(N, V, generator=_gen(31)) * 3).to(torch.bfloat16).to(dev)
    t = torch.randint(0, V, (N, k), generator=_gen(32)).to(dev)
    g = torch.randn(N, k, generator=_gen(33)).to(dev)
    lp, st = rlk.logp_fwd(x, t, 20.0)
    gx = rlk.logp_bwd(x, t, g, st, 20.0)
    out = torch.full_like(lp, float("nan"))
    st2 = torch.zeros_like(st)
    gx2 = torch.full_like(gx, float("nan"))
    fwd = rlk.prepare(rlk.rlk_logp_fwd, x, t, 20.0, out, st2)
    bwd = rlk.prepare(rlk.rlk_logp_bwd, x, t, 20.0, st2, g, gx2)
    for _ in range(3):
        fwd()
        bwd()
    torch.cuda.synchronize()
    assert torch.equal(out, lp) and torch.equal(st2, st) and torch.equal(gx2, gx)
    # the C library still validates each call: a NaN cap is rejected on call
    bad = rlk.prepare(rlk.rlk_logp_fwd, x, t, float("nan"), out, st2)
    with pytest.raises(rlk.RLKError):
        bad()
    with pytest.raises(ValueError):
        rlk.prepare(lambda: None)   # makes no library call
