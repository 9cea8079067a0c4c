"""Vocabulary shards: per-shard partial records, the P-way combine and the
per-shard backward, against the fp64 oracle on the unsharded rows.

The split follows "Add Triton kernels for vocab-parallel logprobs, entropy and
KL" (DeepSpeed pull request 8838, Changes): each shard reduces its own columns
once, the records are rescaled to the global maximum and summed, and every
shard then computes its own gradient columns from the global row record.
Here the P shards are column slices of one tensor on one GPU; the gather of
the records is a plain stack.  Cases: uneven bounds, an empty shard, targets
on shard edges, ignored and out-of-range targets, a row whose whole shard is
masked, empty rows, support mismatch confined to one shard; and a one-shard
combine that must reproduce the plain forward bit for bit.
"""

import numpy as np
import pytest
import torch

from tests.parity import assert_grad, assert_out, to64
from tests.test_parity_gpu import gen, kl_pair, logits_rows
from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.bfloat16]
DT_IDS = ["f32", "bf16"]


def splits(V):
    """Shard bounds: uneven with an empty shard, and eight near-even shards."""
    a, b = V // 3, (3 * V) // 4
    out = [[0, a, a, b, V]]
    if V >= 8:
        out.append([round(i * V / 8) for i in range(9)])
    return out


def _pieces(x, bounds):
    return [x[:, bounds[s]:bounds[s + 1]] for s in range(len(bounds) - 1)]


def sharded_logp(dev, x, t, g, bounds, cap):
    N, V = x.shape
    k = t.shape[1]
    P = len(bounds) - 1
    parts = rlk.new_partials(P, N, dev)
    tv = torch.empty(P, N, k, dtype=torch.float32, device=dev)
    for s, xs in enumerate(_pieces(x, bounds)):
        rlk.rlk_logp_fwd_partial(xs, bounds[s], V, t, cap, parts[s], tv[s])
    out = torch.empty(N, k, dtype=torch.float32, device=dev)
    stats = rlk.new_stats(rlk.RLK_HEAD_LOGP, N, V, dev)
    rlk.rlk_combine(rlk.RLK_HEAD_LOGP, 0, bounds, parts, t, tv, cap, out, stats)
    grads = []
    for s, xs in enumerate(_pieces(x, bounds)):
        gs = torch.full(xs.shape, float("nan"), dtype=x.dtype, device=dev)
        rlk.rlk_logp_bwd_shard(xs, bounds[s], V, t, cap, stats, g, gs)
        grads.append(gs)
    torch.cuda.synchronize()
    return out, stats, torch.cat(grads, 1)


def sharded_entropy(dev, x, g, bounds, cap):
    N, V = x.shape
    P = len(bounds) - 1
    parts = rlk.new_partials(P, N, dev)
    for s, xs in enumerate(_pieces(x, bounds)):
        rlk.rlk_entropy_fwd_partial(xs, cap, parts[s])
    out = torch.empty(N, dtype=torch.float32, device=dev)
    stats = rlk.new_stats(rlk.RLK_HEAD_ENTROPY, N, V, dev)
    rlk.rlk_combine(rlk.RLK_HEAD_ENTROPY, 0, bounds, parts, None, None, cap, out, stats)
    grads = [rlk.entropy_bwd(xs, g, stats, cap) if xs.shape[1] else xs.new_empty(N, 0)
             for xs in _pieces(x, bounds)]
    torch.cuda.synchronize()
    return out, stats, torch.cat(grads, 1)


def sharded_kl(dev, a, b, g, bounds, direction, cp, cr):
    N, V = a.shape
    P = len(bounds) - 1
    parts = rlk.new_partials(P, N, dev)
    for s, (xa, xb) in enumerate(zip(_pieces(a, bounds), _pieces(b, bounds))):
        rlk.rlk_kl_fwd_partial(xa, xb, direction, cp, cr, parts[s])
    out = torch.empty(N, dtype=torch.float32, device=dev)
    stats = rlk.new_stats(rlk.RLK_HEAD_KL, N, V, dev)
    rlk.rlk_combine(rlk.RLK_HEAD_KL, direction, bounds, parts, None, None, 0.0, out, stats)
    grads = [rlk.kl_bwd(xa, xb, g, stats, direction, cp, cr) if xa.shape[1]
             else xa.new_empty(N, 0)
             for xa, xb in zip(_pieces(a, bounds), _pieces(b, bounds))]
    torch.cuda.synchronize()
    return out, stats, torch.cat(grads, 1)


def _bits(t):
    return t.contiguous().view(torch.uint8).cpu()


# ------------------------------------------------------------------ logprobs

@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("V", [7, 1031, 32000])
@pytest.mark.parametrize("k", [1, 40])
@pytest.mark.parametrize("cap", [0.0, 30.0, 50.0])
def test_logp_shards(dev, orc, dtype, V, k, cap):
    N = 10
    for bounds in splits(V):
        x = logits_rows(N, V, 15.0 if cap else 3.0, torch.float32, V + k)
        if not cap:
            x[3] = float("-inf")                          # empty row
            if bounds[3] > bounds[2]:
                x[4, bounds[2]:bounds[3]] = float("-inf")  # one whole shard masked
        x = x.to(dtype)
        t = torch.randint(0, V, (N, k), generator=gen(V * k))
        # targets on shard edges, ignored, out of range, one row fully ignored
        for s in range(len(bounds) - 1):
            if bounds[s] < V:
                t[s % N, (s * 7) % k] = bounds[s]
        t[1, 0] = -100
        t[2, k - 1] = V + 3
        t[6] = -100
        g = torch.randn(N, k, generator=gen(V * k + 1))
        xd, td, gd = x.to(dev), t.to(dev), g.to(dev)
        out, _, gx = sharded_logp(dev, xd, td, gd, bounds, cap)
        x64 = to64(x)
        ign = (t < 0) | (t >= V)
        assert_out(out, orc.logp_fwd(x64, t.numpy(), cap), dtype, f"logp {bounds}",
                   exact_zero=ign.numpy())
        row_zero = np.repeat(ign.all(1).numpy()[:, None], V, 1)
        assert_grad(gx, orc.logp_bwd(x64, t.numpy(), to64(g), cap), f"grad {bounds}",
                    exact_zero=row_zero)


# ------------------------------------------------------------------- entropy

@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("V", [7, 1031, 32000])
@pytest.mark.parametrize("cap", [0.0, 30.0, 50.0])
def test_entropy_shards(dev, orc, dtype, V, cap):
    N = 10
    for bounds in splits(V):
        x = logits_rows(N, V, 15.0 if cap else 3.0, torch.float32, V + 11,
                        masked_frac=0.1 if (V > 2 and not cap) else 0.0)
        if not cap:
            x[3] = float("-inf")
            if bounds[3] > bounds[2]:
                x[4, bounds[2]:bounds[3]] = float("-inf")
        x = x.to(dtype)
        g = torch.randn(N, generator=gen(V + 12))
        out, _, gx = sharded_entropy(dev, x.to(dev), g.to(dev), bounds, cap)
        x64 = to64(x)
        assert_out(out, orc.entropy_fwd(x64, cap), dtype, f"entropy {bounds}")
        ez = None if cap else (np.isneginf(x64) & ~np.isneginf(x64).all(1, keepdims=True))
        assert_grad(gx, orc.entropy_bwd(x64, to64(g), cap), f"entropy grad {bounds}",
                    exact_zero=ez)


# ------------------------------------------------------------------------ KL

@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("V", [7, 1031, 32000])
@pytest.mark.parametrize("direction", [0, 1], ids=["rev", "fwd"])
@pytest.mark.parametrize("caps", [(0.0, 0.0), (30.0, 20.0)], ids=["nocap", "cap"])
def test_kl_shards(dev, orc, dtype, V, direction, caps):
    N = 12
    cp, cr = caps
    for bounds in splits(V):
        a, b = kl_pair(N, V, torch.float32, V + 21, mismatch_rows=(1,) if not cr else (),
                       empty_rows=(3,) if not (cp or cr) else (),
                       both_masked_rows=(5,) if not (cp or cr) else (),
                       underflow_row=7 if not (cp or cr) else None)
        if not (cp or cr) and bounds[3] > bounds[2]:
            a[8, bounds[2]:bounds[3]] = float("-inf")     # a whole shard masked on both
            b[8, bounds[2]:bounds[3]] = float("-inf")
        if not cr:
            b[9] = float("-inf")                            # empty reference only
        a, b = a.to(dtype), b.to(dtype)
        g = torch.randn(N, generator=gen(V + 22))
        out, _, gx = sharded_kl(dev, a.to(dev), b.to(dev), g.to(dev), bounds, direction, cp, cr)
        a64, b64 = to64(a), to64(b)
        assert_out(out, orc.kl_fwd(a64, b64, direction, cp, cr), dtype, f"kl {bounds}")
        assert_grad(gx, orc.kl_bwd(a64, b64, to64(g), direction, cp, cr), f"kl grad {bounds}")


# ------------------------------------------------- one shard == plain forward

@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("cap", [0.0, 20.0, 60.0])
def test_single_shard_combine_is_bitwise_plain(dev, dtype, cap):
    N, V, k = 9, 4099, 5
    x = logits_rows(N, V, 6.0, dtype, 3).to(dev)
    y = logits_rows(N, V, 6.0, dtype, 4).to(dev)
    t = torch.randint(-2, V + 2, (N, k), generator=gen(5)).to(dev)
    bounds = [0, V]
    parts = rlk.new_partials(1, N, dev)
    tv = torch.empty(1, N, k, dtype=torch.float32, device=dev)

    want_lp, want_st = rlk.logp_fwd(x, t, cap)
    rlk.rlk_logp_fwd_partial(x, 0, V, t, cap, parts[0], tv[0])
    lp = torch.empty(N, k, dtype=torch.float32, device=dev)
    st = rlk.new_stats(rlk.RLK_HEAD_LOGP, N, V, dev)
    rlk.rlk_combine(rlk.RLK_HEAD_LOGP, 0, bounds, parts, t, tv, cap, lp, st)
    assert torch.equal(_bits(lp), _bits(want_lp)) and torch.equal(_bits(st), _bits(want_st))

    want_h, want_st = rlk.entropy_fwd(x, cap)
    rlk.rlk_entropy_fwd_partial(x, cap, parts[0])
    h = torch.empty(N, dtype=torch.float32, device=dev)
    rlk.rlk_combine(rlk.RLK_HEAD_ENTROPY, 0, bounds, parts, None, None, cap, h, st)
    assert torch.equal(_bits(h), _bits(want_h)) and torch.equal(_bits(st), _bits(want_st))

    for d in (0, 1):
        want_d, want_st = rlk.kl_fwd(x, y, d, cap, 0.0)
        rlk.rlk_kl_fwd_partial(x, y, d, cap, 0.0, parts[0])
        D = torch.empty(N, dtype=torch.float32, device=dev)
        rlk.rlk_combine(rlk.RLK_HEAD_KL, d, bounds, parts, None, None, 0.0, D, st)
        assert torch.equal(_bits(D), _bits(want_d)) and torch.equal(_bits(st), _bits(want_st))


def test_shard_backward_equals_plain_backward_columns(dev):
    # with the same row record, a shard's gradient is exactly the plain
    # gradient's columns (the backward is elementwise given the record)
    N, V, k = 7, 9000, 3
    x = logits_rows(N, V, 4.0, torch.bfloat16, 8).to(dev)
    t = torch.randint(0, V, (N, k), generator=gen(9)).to(dev)
    g = torch.randn(N, k, generator=gen(10)).to(dev)
    lp, st = rlk.logp_fwd(x, t)
    want = rlk.logp_bwd(x, t, g, st)
    for b0, b1 in [(0, 3001), (3001, 3001), (3001, 9000), (17, 4113)]:
        gs = torch.empty(N, b1 - b0, dtype=x.dtype, device=dev)
        rlk.rlk_logp_bwd_shard(x[:, b0:b1], b0, V, t, 0.0, st, g, gs)
        torch.cuda.synchronize()
        assert torch.equal(_bits(gs), _bits(want[:, b0:b1])), (b0, b1)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_table_forward_partials(dev, dtype):
    # Shards wide enough for the fixed cap's odd form in both heads: in a
    # call of 1030 rows the LDS-table forward writes the partial records, in
    # a 65-row subset the computed form does.  Records, target inputs and
    # combined heads agree bit for bit; one shard's combine equals the plain
    # call bit for bit; two shards match the plain call.
    N, W, k, cap = 1030, 196616, 3, 20.0
    V = 2 * W
    g = torch.Generator(device=dev).manual_seed(31)
    x = (torch.randn(N, V, generator=g, device=dev) * 4).to(dtype)
    t = torch.randint(-2, V + 2, (N, k), generator=g, device=dev)
    bounds = [0, W, V]
    sub = torch.arange(0, N, 16, device=dev)

    def run(xx, tt):
        n = xx.shape[0]
        parts = rlk.new_partials(2, n, dev)
        eparts = rlk.new_partials(2, n, dev)
        tv = torch.empty(2, n, k, dtype=torch.float32, device=dev)
        for s in range(2):
            xs = xx[:, bounds[s]:bounds[s + 1]]
            rlk.rlk_logp_fwd_partial(xs, bounds[s], V, tt, cap, parts[s], tv[s])
            rlk.rlk_entropy_fwd_partial(xs, cap, eparts[s])
        lp = torch.empty(n, k, dtype=torch.float32, device=dev)
        st = rlk.new_stats(rlk.RLK_HEAD_LOGP, n, V, dev)
        rlk.rlk_combine(rlk.RLK_HEAD_LOGP, 0, bounds, parts, tt, tv, cap, lp, st)
        h = torch.empty(n, dtype=torch.float32, device=dev)
        sh = rlk.new_stats(rlk.RLK_HEAD_ENTROPY, n, V, dev)
        rlk.rlk_combine(rlk.RLK_HEAD_ENTROPY, 0, bounds, eparts, None, None, cap, h, sh)
        torch.cuda.synchronize()
        return {"parts": parts[:, :n * 32].reshape(2, n, 32), "eparts": eparts[:, :n * 32].reshape(2, n, 32),
                "tv": tv, "lp": lp, "st": st.view(n, -1), "h": h, "sh": sh.view(n, -1)}

    full = run(x, t)
    part = run(x[sub].contiguous(), t[sub].contiguous())
    for key in full:
        a = full[key][:, sub] if key in ("parts", "eparts", "tv") else full[key][sub]
        assert torch.equal(_bits(a), _bits(part[key])), key
    lp0, _ = rlk.logp_fwd(x, t, cap)
    h0, _ = rlk.entropy_fwd(x, cap)
    torch.testing.assert_close(full["lp"], lp0, rtol=0, atol=2e-4)
    torch.testing.assert_close(full["h"], h0, rtol=1e-5, atol=1e-5)
    del full, part

    x1 = x[:, :W].contiguous()
    t1 = torch.randint(0, W, (N, k), generator=g, device=dev)
    want_lp, want_st = rlk.logp_fwd(x1, t1, cap)
    parts = rlk.new_partials(1, N, dev)
    tv = torch.empty(1, N, k, dtype=torch.float32, device=dev)
    rlk.rlk_logp_fwd_partial(x1, 0, W, t1, cap, parts[0], tv[0])
    lp = torch.empty(N, k, dtype=torch.float32, device=dev)
    st = rlk.new_stats(rlk.RLK_HEAD_LOGP, N, W, dev)
    rlk.rlk_combine(rlk.RLK_HEAD_LOGP, 0, [0, W], parts, t1, tv, cap, lp, st)
    assert torch.equal(_bits(lp), _bits(want_lp)) and torch.equal(_bits(st), _bits(want_st))
    want_h, want_sh = rlk.entropy_fwd(x1, cap)
    rlk.rlk_entropy_fwd_partial(x1, cap, parts[0])
    h = torch.empty(N, dtype=torch.float32, device=dev)
    sh = rlk.new_stats(rlk.RLK_HEAD_ENTROPY, N, W, dev)
    rlk.rlk_combine(rlk.RLK_HEAD_ENTROPY, 0, [0, W], parts, None, None, cap, h, sh)
    assert torch.equal(_bits(h), _bits(want_h)) and torch.equal(_bits(sh), _bits(want_sh))
