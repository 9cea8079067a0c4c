"""The five measured workloads at full size, checked against the oracle.

Each workload is generated on the GPU at its real shape (up to bf16
[32768, 151936], 10 GB) and run forward + backward through the C ABI in the
same launch configuration the benchmark times.  Rows are independent, so the
oracle recomputes a sample of rows one by one: every special row (ignored or
out-of-range targets, support-mismatch rows, all -inf rows, +1000 offset rows,
fully ignored top-k rows) plus seeded random rows, the first and the last.
Everything the test compares is a whole row.
"""

import math

import numpy as np
import pytest
import torch

from tests.parity import assert_grad, assert_out, strict_bf16_misses, to64
from vocab_log_softmax_amd import rlk, workloads

pytestmark = pytest.mark.gpu


def sample_rows(N, special, n_random=24, seed=0):
    g = torch.Generator().manual_seed(seed)
    rnd = torch.randperm(N, generator=g)[:n_random].tolist()
    rows = set(rnd) | {0, N - 1}
    for s in special:
        rows |= set(int(r) for r in s)
    return sorted(rows)


def free_after(*ts):
    for t in ts:
        del t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["c1_logp_fp32", "c2_logp_bf16", "c5_topk_cap20"])
def test_logp_workload(dev, orc, name):
    d = workloads.make_inputs(name, dev)
    w = d["workload"]
    x, t, g = d["logits"], d["targets"], d["grad"]
    N, V = x.shape
    out, st = rlk.logp_fwd(x, t, w.cap)
    gx = rlk.logp_bwd(x, t, g, st, w.cap)
    torch.cuda.synchronize()
    special = [d.get("ignored_rows", []), d.get("oob_rows", [])]
    rows = sample_rows(N, special, seed=w.seed) if N > 64 else list(range(N))
    ri = torch.tensor(rows, device=dev)
    x64 = to64(x[ri])
    t_np = t[ri].cpu().numpy()
    g64 = to64(g[ri])
    ref = orc.logp_fwd(x64, t_np, w.cap)
    refg = orc.logp_bwd(x64, t_np, g64, w.cap)
    ign = (t_np < 0) | (t_np >= V)
    assert_out(out[ri], ref, x.dtype, f"{name} logp", exact_zero=ign)
    assert_grad(gx[ri], refg, f"{name} grad",
                exact_zero=np.repeat(ign.all(1)[:, None], V, 1))
    if x.dtype == torch.bfloat16:
        print(f"{name}: {strict_bf16_misses(gx[ri], refg)} gradient elements above the strict "
              f"4e-3 bound (each within half a bf16 ulp plus the fp32 slack)")
    # every ignored slot of the whole batch is exactly 0, not just the sample
    all_ign = (t < 0) | (t >= V)
    assert bool((out[all_ign] == 0).all())
    full_ign_rows = all_ign.all(1)
    if bool(full_ign_rows.any()):
        assert bool((gx[full_ign_rows] == 0).all())


def test_kl_workload(dev, orc):
    name = "c3_kl_bf16"
    d = workloads.make_inputs(name, dev)
    a, b, g = d["logits"], d["ref"], d["grad"]
    N, V = a.shape
    rows = sample_rows(N, [d["mismatch_rows"], d["empty_rows"]], seed=3)
    ri = torch.tensor(rows, device=dev)
    a64, b64, g64 = to64(a[ri]), to64(b[ri]), to64(g[ri])
    for direction in (0, 1):
        D, st = rlk.kl_fwd(a, b, direction)
        gx = rlk.kl_bwd(a, b, g, st, direction)
        torch.cuda.synchronize()
        ref = orc.kl_fwd(a64, b64, direction)
        refg = orc.kl_bwd(a64, b64, g64, direction)
        assert_out(D[ri], ref, a.dtype, f"KL dir={direction}")
        assert_grad(gx[ri], refg, f"KL grad dir={direction}")
        # structure over the whole batch: mismatch rows +inf (reverse) / finite (forward)
        mis = d["mismatch_rows"].to(dev)
        emp = d["empty_rows"].to(dev)
        if direction == 0:
            assert bool(torch.isposinf(D[mis]).all())
        else:
            assert bool(torch.isfinite(D[mis]).all())
        assert bool(torch.isnan(D[emp]).all())
        del gx, st
        torch.cuda.empty_cache()


def test_entropy_workload(dev, orc):
    name = "c4_entropy_cap30"
    d = workloads.make_inputs(name, dev)
    w = d["workload"]
    x, g = d["logits"], d["grad"]
    N, V = x.shape
    H, st = rlk.entropy_fwd(x, w.cap)
    gx = rlk.entropy_bwd(x, g, st, w.cap)
    torch.cuda.synchronize()
    rows = sample_rows(N, [d["offset_rows"][:16]], n_random=16, seed=4)
    ri = torch.tensor(rows, device=dev)
    x64 = to64(x[ri])
    assert_out(H[ri], orc.entropy_fwd(x64, w.cap), x.dtype, "entropy")
    assert_grad(gx[ri], orc.entropy_bwd(x64, to64(g[ri]), w.cap), "entropy grad")
    # all 64 offset rows saturate the cap: uniform rows, H = log V
    off = d["offset_rows"].to(dev)
    assert np.allclose(to64(H[off]), math.log(V), atol=2e-3)


def test_standalone_softcap_workload(dev, orc):
    x, gy = workloads.make_softcap_inputs("c5_topk_cap20", dev)
    for cap in (20.0, 30.0):
        y = rlk.softcap_fwd(x, cap)
        gx = rlk.softcap_bwd(x, gy, cap)
        torch.cuda.synchronize()
        x64 = to64(x).reshape(-1)
        ry = orc.softcap_fwd(x64, cap)
        yy = to64(y).reshape(-1)
        assert (np.abs(yy - ry) <= 1e-5 * np.abs(ry) + 1e-30).all()
        assert_grad(gx.reshape(-1), orc.softcap_bwd(x64, to64(gy).reshape(-1), cap),
                    "softcap grad")
