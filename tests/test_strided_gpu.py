"""Two-stride row views ([B, T, V] with strides (sB, sT, 1)) read in place.

The pages' patch addresses rows with two strides so that a sequence slice such
as logits[:, :-1] is not copied, and tests it with NaN in every position
outside the view ("Add Triton kernels for vocab-parallel logprobs, entropy and
KL", review comment).  Here the strided entry points must give bitwise the
same outputs and gradients as the plain entry points on a contiguous copy,
must never read the poisoned positions, and can write the gradient straight
into the slice of a full [B, T + 1, V] buffer without touching the rest.
"""

import pytest
import torch

from tests.test_invariance_gpu import assert_bitwise
from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu


def _gen(seed):
    return torch.Generator().manual_seed(seed)


def all_heads(x, ref, t, g_t, g_r, cap, out_bufs=None):
    """Every head on x (2-D or 3-D); grads optionally written into given views."""
    res = {}
    lp, st = rlk.logp_fwd(x, t, cap)
    res["logp"] = lp.reshape(-1, t.shape[-1])
    o = None if out_bufs is None else out_bufs[0]
    res["logp_grad"] = rlk.logp_bwd(x, t, g_t, st, cap, out=o) if x.dim() == 3 else \
        rlk.logp_bwd(x, t, g_t, st, cap)
    h, st = rlk.entropy_fwd(x, cap)
    res["ent"] = h.reshape(-1)
    o = None if out_bufs is None else out_bufs[1]
    res["ent_grad"] = rlk.entropy_bwd(x, g_r, st, cap, out=o) if x.dim() == 3 else \
        rlk.entropy_bwd(x, g_r, st, cap)
    for d in (0, 1):
        k, st = rlk.kl_fwd(x, ref, d, cap, 0.0)
        res[f"kl{d}"] = k.reshape(-1)
        o = None if out_bufs is None else out_bufs[2 + d]
        res[f"kl{d}_grad"] = rlk.kl_bwd(x, ref, g_r, st, d, cap, 0.0, out=o) if x.dim() == 3 \
            else rlk.kl_bwd(x, ref, g_r, st, d, cap, 0.0)
    torch.cuda.synchronize()
    return res


def make_seq(B, T1, V, dtype, seed, dev):
    x = (torch.randn(B, T1, V, generator=_gen(seed)) * 4).to(dtype).to(dev)
    ref = (x.float() + torch.randn(B, T1, V, generator=_gen(seed + 1)).to(dev) * 0.5).to(dtype)
    x[0, 1, : V // 4] = float("-inf")
    ref[0, 1, : V // 4] = float("-inf")
    return x, ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16],
                         ids=["bf16", "f32", "f16"])
@pytest.mark.parametrize("V", [4096, 32000, 4099])
@pytest.mark.parametrize("cap", [0.0, 30.0, 50.0])
@pytest.mark.parametrize("k", [2, 40])  # one-shot pieces / wide top-k pieces
def test_sequence_slice_in_place(dev, dtype, V, cap, k):
    B, T1 = 3, 9
    T = T1 - 1
    x, ref = make_seq(B, T1, V, dtype, V, dev)
    # the position outside the view is poisoned: reading it would leak NaN
    x[:, -1] = float("nan")
    ref[:, -1] = float("nan")
    xv, rv = x[:, :-1], ref[:, :-1]
    assert not xv.is_contiguous()
    t = torch.randint(0, V, (B * T, k), generator=_gen(2)).to(dev)
    t[3, 0] = -100
    t[5, k - 1] = t[5, 0]
    g_t = torch.randn(B * T, k, generator=_gen(3)).to(dev)
    g_r = torch.randn(B * T, generator=_gen(4)).to(dev)
    want = all_heads(xv.reshape(B * T, V).contiguous(), rv.reshape(B * T, V).contiguous(),
                     t, g_t, g_r, cap)
    got = all_heads(xv, rv, t, g_t, g_r, cap)
    for key in want:
        assert_bitwise(want[key], got[key].reshape(want[key].shape), f"slice {key}")


def test_gradient_written_into_a_slice_of_the_full_buffer(dev):
    B, T1, V = 2, 6, 5000
    T = T1 - 1
    x, ref = make_seq(B, T1, V, torch.bfloat16, 11, dev)
    xv, rv = x[:, :-1], ref[:, :-1]
    t = torch.randint(0, V, (B * T, 1), generator=_gen(5)).to(dev)
    g_t = torch.randn(B * T, 1, generator=_gen(6)).to(dev)
    g_r = torch.randn(B * T, generator=_gen(7)).to(dev)
    sentinel = 7.0
    bufs = [torch.full((B, T1, V), sentinel, dtype=torch.bfloat16, device=dev) for _ in range(4)]
    got = all_heads(xv, rv, t, g_t, g_r, 0.0, out_bufs=[b[:, :-1] for b in bufs])
    want = all_heads(xv.reshape(B * T, V).contiguous(), rv.reshape(B * T, V).contiguous(),
                     t, g_t, g_r, 0.0)
    for b, key in zip(bufs, ["logp_grad", "ent_grad", "kl0_grad", "kl1_grad"]):
        assert_bitwise(want[key].reshape(B, T, V), b[:, :-1].contiguous(), f"in-place {key}")
        assert bool((b[:, -1] == sentinel).all()), f"{key} wrote outside its slice"
        assert got[key].data_ptr() == b.data_ptr()


def test_time_major_view(dev):
    # a [T, B, V] tensor seen as [B, T, V]: row stride B*V, batch stride V
    T, B, V = 7, 4, 8192
    base = (torch.randn(T, B, V, generator=_gen(8)) * 3).to(torch.bfloat16).to(dev)
    rbase = (base.float() + 0.3).to(torch.bfloat16)
    xv, rv = base.transpose(0, 1), rbase.transpose(0, 1)
    t = torch.randint(0, V, (B * T, 1), generator=_gen(9)).to(dev)
    g_t = torch.randn(B * T, 1, generator=_gen(10)).to(dev)
    g_r = torch.randn(B * T, generator=_gen(11)).to(dev)
    want = all_heads(xv.reshape(B * T, V).contiguous(), rv.reshape(B * T, V).contiguous(),
                     t, g_t, g_r, 20.0)
    got = all_heads(xv, rv, t, g_t, g_r, 20.0)
    for key in want:
        assert_bitwise(want[key], got[key].reshape(want[key].shape), f"time-major {key}")


def test_autograd_on_a_slice(dev):
    B, T1, V = 2, 5, 3000
    x = (torch.randn(B, T1, V, generator=_gen(12)) * 3).to(dev).requires_grad_(True)
    t = torch.randint(0, V, (B, T1 - 1), generator=_gen(13)).to(dev)
    lp = rlk.logprobs(x[:, :-1], t)
    lp.sum().backward()
    ref = torch.log_softmax(x.detach()[:, :-1].double(), -1).gather(-1, t[..., None])[..., 0]
    assert torch.allclose(lp.double(), ref, atol=1e-5, rtol=1e-5)
    assert bool((x.grad[:, -1] == 0).all())
    p = torch.softmax(x.detach()[:, :-1].double(), -1)
    onehot = torch.zeros_like(p).scatter_(-1, t[..., None], 1.0)
    assert torch.allclose(x.grad[:, :-1].double(), onehot - p, atol=1e-5)
