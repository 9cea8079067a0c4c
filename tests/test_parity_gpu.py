"""HIP path vs the fp64 oracle, element by element, on small seeded inputs.

Shapes span several 2048-element tiles and ragged tails (V = 1, 2, 7, 255,
1031, 4097, 32000, ...), both dtypes, with and without the softcap, and the
special rows the pages list: masked columns, all -inf rows, ignored and
out-of-range targets, duplicate top-k ids, fully ignored rows, support
mismatch (with an underflowing probability), +1000 offsets, saturation.
All calls go through the C ABI (the ctypes binding).
"""

import math

import numpy as np
import pytest
import torch

from tests.parity import assert_grad, assert_out, to64
from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu

VS = [1, 2, 7, 255, 1031, 2048, 4097, 32000]
DTYPES = [torch.float32, torch.bfloat16, torch.float16]
DT_IDS = ["f32", "bf16", "f16"]


def gen(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def logits_rows(N, V, std, dtype, seed, masked_frac=0.0, empty_rows=(), offset_rows=(),
                offset=1000.0):
    g = gen(seed)
    x = torch.randn(N, V, generator=g) * std
    for r in offset_rows:
        x[r] += offset
    if masked_frac:
        m = torch.rand(N, V, generator=g) < masked_frac
        keep = torch.randint(0, V, (N,), generator=g)
        m[torch.arange(N), keep] = False
        x[m] = float("-inf")
    for r in empty_rows:
        x[r] = float("-inf")
    return x.to(dtype)


# ------------------------------------------------------------------ logprobs

def _run_logp(dev, orc, x, t, g, cap):
    xd, td, gd = x.to(dev), t.to(dev), g.to(dev)
    out, stats = rlk.logp_fwd(xd, td, cap)
    gx = rlk.logp_bwd(xd, td, gd, stats, cap)
    torch.cuda.synchronize()
    x64 = to64(x)
    ref_out = orc.logp_fwd(x64, t.numpy(), cap)
    ref_gx = orc.logp_bwd(x64, t.numpy(), to64(g), cap)
    return out, gx, ref_out, ref_gx


# Caps 20 and 30 take the fixed-reference form of the fused cap, 50 and 60
# (2 c log2 e above 120) the running-max form.
@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("V", VS)
@pytest.mark.parametrize("cap", [0.0, 30.0, 50.0])
def test_logp_k1(dev, orc, dtype, V, cap):
    N = 12
    x = logits_rows(N, V, 3.0 if not cap else 15.0, dtype, V,
                    masked_frac=0.1 if (V > 2 and not cap) else 0.0,
                    empty_rows=(3,) if not cap else (), offset_rows=(5,))
    t = torch.randint(0, V, (N, 1), generator=gen(V + 1))
    t[1, 0] = -100
    t[2, 0] = V + 7
    t[4, 0] = -1
    g = torch.randn(N, 1, generator=gen(V + 2))
    out, gx, ref_out, ref_gx = _run_logp(dev, orc, x, t, g, cap)
    ignored = (t[:, 0] < 0) | (t[:, 0] >= V)
    assert_out(out, ref_out, dtype, "logp", exact_zero=ignored.numpy()[:, None])
    assert_grad(gx, ref_gx, "grad", exact_zero=np.repeat(ignored.numpy()[:, None], V, 1))


def test_logp_empty_row_without_valid_target_is_zero(dev, orc):
    V = 300
    x = logits_rows(3, V, 3.0, torch.bfloat16, 0, empty_rows=(0, 1))
    t = torch.tensor([[-100], [5], [7]])
    g = torch.tensor([[1.0], [2.0], [3.0]])
    out, gx, ref_out, ref_gx = _run_logp(dev, orc, x, t, g, 0.0)
    assert to64(out)[0, 0] == 0 and math.isnan(to64(out)[1, 0])
    assert (to64(gx)[0] == 0).all() and np.isnan(to64(gx)[1]).all()
    assert_out(out, ref_out, torch.bfloat16)
    assert_grad(gx, ref_gx)


def test_logp_target_on_masked_column(dev, orc):
    V = 1000
    x = logits_rows(2, V, 3.0, torch.float32, 1)
    x[0, 17] = float("-inf")
    t = torch.tensor([[17], [3]])
    g = torch.tensor([[1.5], [1.0]])
    out, gx, ref_out, ref_gx = _run_logp(dev, orc, x, t, g, 0.0)
    assert to64(out)[0, 0] == -np.inf
    assert to64(gx)[0, 17] == 1.5
    assert_out(out, ref_out, torch.float32)
    assert_grad(gx, ref_gx)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("V,k", [(7, 4), (255, 17), (4097, 64), (14000, 64), (32768, 256),
                                 (2000, 300), (20000, 1024), (3000, 4096)])
@pytest.mark.parametrize("cap", [0.0, 20.0, 60.0])
def test_logp_topk(dev, orc, dtype, V, k, cap):
    N = 9
    x = logits_rows(N, V, 10.0 if cap else 3.0, dtype, V + k)
    t = torch.randint(0, V, (N, k), generator=gen(k))
    gsel = gen(k + 1)
    # duplicates, ignored ids, out-of-range ids, one fully ignored row
    for r in range(N):
        for _ in range(max(1, k // 20)):
            j, jj = torch.randint(0, k, (2,), generator=gsel).tolist()
            t[r, j] = t[r, jj]
        for _ in range(max(1, k // 20)):
            j = int(torch.randint(0, k, (1,), generator=gsel))
            t[r, j] = -100
    t[2, 0] = V
    t[6] = -100
    g = torch.randn(N, k, generator=gen(k + 2))
    out, gx, ref_out, ref_gx = _run_logp(dev, orc, x, t, g, cap)
    ign = ((t < 0) | (t >= V)).numpy()
    assert_out(out, ref_out, dtype, "topk logp", exact_zero=ign)
    row_zero = np.repeat(ign.all(1)[:, None], V, 1)
    assert_grad(gx, ref_gx, "topk grad", exact_zero=row_zero)


# ------------------------------------------------------------------- entropy

@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("V", VS)
@pytest.mark.parametrize("cap", [0.0, 30.0, 50.0])
def test_entropy(dev, orc, dtype, V, cap):
    N = 10
    x = logits_rows(N, V, 15.0 if cap else 3.0, dtype, 100 + V,
                    masked_frac=0.1 if (V > 2 and not cap) else 0.0,
                    empty_rows=(2,) if not cap else (), offset_rows=(4, 7))
    x[8] = 0.5                                   # uniform row: H = log V
    xd = x.to(dev)
    g = torch.randn(N, generator=gen(V))
    H, stats = rlk.entropy_fwd(xd, cap)
    gx = rlk.entropy_bwd(xd, g.to(dev), stats, cap)
    torch.cuda.synchronize()
    x64 = to64(x)
    assert_out(H, orc.entropy_fwd(x64, cap), dtype, "entropy")
    masked = np.isneginf(x64) & ~np.isneginf(x64).all(1, keepdims=True) if not cap else None
    assert_grad(gx, orc.entropy_bwd(x64, to64(g), cap), "entropy grad", exact_zero=masked)


@pytest.mark.parametrize("cap", [41.5, 41.7], ids=["fixed_edge", "online_edge"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_cap_mode_edge_rows(dev, orc, cap, dtype):
    """Both sides of the cap-form threshold (2 c log2 e = 120 lies between the
    two caps) on rows at the ends of the cap: every logit far below (all
    shifted exponents near -2 c log2 e, the smallest row sums of the fixed
    form), -inf and +inf columns (slope exactly 0), all at +1000, mixed."""
    N, V = 8, 4097
    x = torch.randn(N, V, generator=gen(11)) * 15.0
    x[0] = -1e4
    x[1] = float("-inf")
    x[2, :5] = float("inf")
    x[2, 5:10] = float("-inf")
    x[3] += 1000.0
    x[4, ::2] = -1e4
    x[5, :V // 2] = float("-inf")
    x = x.to(dtype)
    inf_cols = np.isinf(to64(x))
    xd = x.to(dev)
    t = torch.randint(0, V, (N, 1), generator=gen(12))
    t[2, 0] = 1                                   # a +inf column
    t[5, 0] = 0                                   # a -inf column
    g = torch.randn(N, 1, generator=gen(13))
    out, gx, ref_out, ref_gx = _run_logp(dev, orc, x, t, g, cap)
    assert_out(out, ref_out, dtype, "logp")
    assert_grad(gx, ref_gx, "logp grad", exact_zero=inf_cols)
    gr = torch.randn(N, generator=gen(14))
    H, st = rlk.entropy_fwd(xd, cap)
    gH = rlk.entropy_bwd(xd, gr.to(dev), st, cap)
    y = (x.double() + torch.randn(N, V, generator=gen(15)) * 0.5).to(dtype)
    y[1] = -1e4
    for d in (0, 1):
        D, sk = rlk.kl_fwd(xd, y.to(dev), d, cap, cap)
        gD = rlk.kl_bwd(xd, y.to(dev), gr.to(dev), sk, d, cap, cap)
        torch.cuda.synchronize()
        assert_out(D, orc.kl_fwd(to64(x), to64(y), d, cap, cap), dtype, f"kl {d}")
        assert_grad(gD, orc.kl_bwd(to64(x), to64(y), to64(gr), d, cap, cap), f"kl {d} grad",
                    exact_zero=inf_cols)
    torch.cuda.synchronize()
    assert_out(H, orc.entropy_fwd(to64(x), cap), dtype, "entropy")
    assert_grad(gH, orc.entropy_bwd(to64(x), to64(gr), cap), "entropy grad", exact_zero=inf_cols)


@pytest.mark.parametrize("cap", [1e-7, 1e-5, 200.0], ids=["tiny", "fixed_min", "large"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_cap_extremes(dev, orc, cap, dtype):
    """Caps far from the usual 20-50: a tiny cap (running-max form below the
    fixed form's lower bound; every logit saturates to +-c), one just inside
    the fixed form's range, and a large cap (y ~ x over the logits' range)."""
    N, V = 6, 3001
    x = (torch.randn(N, V, generator=gen(41)) * 3.0).to(dtype)
    x64 = to64(x)
    t = torch.randint(0, V, (N, 2), generator=gen(42))
    gt = torch.randn(N, 2, generator=gen(43))
    gr = torch.randn(N, generator=gen(44))
    xd = x.to(dev)
    lp, st = rlk.logp_fwd(xd, t.to(dev), cap)
    glp = rlk.logp_bwd(xd, t.to(dev), gt.to(dev), st, cap)
    H, sh = rlk.entropy_fwd(xd, cap)
    gH = rlk.entropy_bwd(xd, gr.to(dev), sh, cap)
    torch.cuda.synchronize()
    assert_out(lp, orc.logp_fwd(x64, t.numpy(), cap), dtype, "logp")
    assert_grad(glp, orc.logp_bwd(x64, t.numpy(), to64(gt), cap), "logp grad")
    assert_out(H, orc.entropy_fwd(x64, cap), dtype, "entropy")
    assert_grad(gH, orc.entropy_bwd(x64, to64(gr), cap), "entropy grad")


def test_entropy_saturated_cap_rows(dev, orc):
    # every logit caps to exactly c: a uniform row, H = log V
    V = 151936
    x = (torch.randn(3, V, generator=gen(9)) * 15 + 1000).to(torch.bfloat16)
    H, stats = rlk.entropy_fwd(x.to(dev), 30.0)
    torch.cuda.synchronize()
    assert np.allclose(to64(H), math.log(V), atol=2e-6)
    assert_out(H, orc.entropy_fwd(to64(x), 30.0), torch.bfloat16)


# ------------------------------------------------------------------------ KL

def kl_pair(N, V, dtype, seed, mismatch_rows=(), empty_rows=(), both_masked_rows=(),
            underflow_row=None, caps=(0.0, 0.0)):
    a = logits_rows(N, V, 3.0, torch.float32, seed)
    b = a + torch.randn(N, V, generator=gen(seed + 1)) * 0.5
    ncols = max(1, math.ceil(0.1 * V))
    for r in mismatch_rows:
        b[r, V - ncols:] = float("-inf")
    for r in both_masked_rows:
        a[r, :ncols] = float("-inf")
        b[r, :ncols] = float("-inf")
    if underflow_row is not None and V >= 3:
        a[underflow_row, 1] = a[underflow_row].max() - 800.0
        b[underflow_row, 1] = float("-inf")
    for r in empty_rows:
        a[r] = float("-inf")
        b[r] = float("-inf")
    return a.to(dtype), b.to(dtype)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("V", [2, 7, 1031, 4097, 32000])
@pytest.mark.parametrize("direction", [0, 1], ids=["rev", "fwd"])
@pytest.mark.parametrize("caps", [(0.0, 0.0), (30.0, 20.0), (50.0, 20.0), (0.0, 45.0), (41.5, 0.0)],
                         ids=["nocap", "cap", "online_fixed", "none_online", "fixed_none"])
def test_kl(dev, orc, dtype, V, direction, caps):
    N = 12
    cp, cr = caps
    a, b = kl_pair(N, V, dtype, V, mismatch_rows=(1,) if not cr else (),
                   empty_rows=(3,) if not (cp or cr) else (),
                   both_masked_rows=(5,) if not (cp or cr) else (),
                   underflow_row=7 if not (cp or cr) else None)
    b[9] = float("-inf") if not cr else b[9]      # empty reference only
    g = torch.randn(N, generator=gen(V + 5))
    ad, bd = a.to(dev), b.to(dev)
    D, stats = rlk.kl_fwd(ad, bd, direction, cp, cr)
    gx = rlk.kl_bwd(ad, bd, g.to(dev), stats, direction, cp, cr)
    torch.cuda.synchronize()
    a64, b64 = to64(a), to64(b)
    assert_out(D, orc.kl_fwd(a64, b64, direction, cp, cr), dtype, "kl")
    ez = None
    if direction == 0 and not cp:
        ez = np.isneginf(a64) & ~np.isneginf(a64).all(1, keepdims=True)
        ez &= ~np.isneginf(b64).all(1, keepdims=True)
    assert_grad(gx, orc.kl_bwd(a64, b64, to64(g), direction, cp, cr), "kl grad", exact_zero=ez)


def test_kl_self_is_zero(dev):
    x = logits_rows(6, 5000, 3.0, torch.bfloat16, 3, masked_frac=0.05).to(dev)
    for d in (0, 1):
        D, stats = rlk.kl_fwd(x, x, d)
        gx = rlk.kl_bwd(x, x, torch.ones(6, device=dev), stats, d)
        torch.cuda.synchronize()
        assert (to64(D) == 0).all()
        assert (to64(gx) == 0).all()


# ------------------------------------------------------------------- softcap

@pytest.mark.parametrize("xdt", DTYPES, ids=["x_" + i for i in DT_IDS])
@pytest.mark.parametrize("ydt", DTYPES, ids=["y_" + i for i in DT_IDS])
@pytest.mark.parametrize("n", [1, 7, 8, 1025, 6921, 6 * 262144])
@pytest.mark.parametrize("cap", [20.0, 30.0])
def test_softcap(dev, orc, xdt, ydt, n, cap):
    g = gen(n)
    x = torch.randn(n, generator=g) * cap * torch.tensor([0.001, 0.3, 1.0, 3.0])[
        torch.randint(0, 4, (n,), generator=g)]
    x[: min(n, 3)] = torch.tensor([float("-inf"), 40 * cap, 0.0])[: min(n, 3)]
    x = x.to(xdt)
    gy = torch.randn(n, generator=g)
    xd = x.to(dev)
    y = rlk.softcap_fwd(xd, cap, ydt)
    gx = rlk.softcap_bwd(xd, gy.to(dev), cap)
    torch.cuda.synchronize()
    x64 = to64(x)
    ry = orc.softcap_fwd(x64, cap)
    if ydt == torch.float32:
        gyv, ryv = to64(y), ry
        fin = np.isfinite(ryv)
        assert (np.abs(gyv[fin] - ryv[fin]) <= 1e-5 * np.abs(ryv[fin]) + 1e-30).all(), \
            np.max(np.abs(gyv[fin] - ryv[fin]) / np.maximum(np.abs(ryv[fin]), 1e-30))
    else:
        assert_grad(y, ry, "softcap y bf16")
    assert_grad(gx, orc.softcap_bwd(x64, to64(gy), cap), "softcap grad")


def test_softcap_shapes_and_views(dev):
    x = (torch.randn(2, 3, 1000) * 25).to(torch.bfloat16).to(dev)
    y = rlk.softcap(x, 30.0)
    assert y.shape == x.shape and y.dtype == torch.float32
    y2 = rlk.softcap_fwd(x[:, 1:], 30.0)          # non-contiguous view is copied first
    torch.cuda.synchronize()
    assert torch.equal(y2, y[:, 1:])
