"""The C ABI under HIP graph capture (GPU).

No entry point allocates, synchronises or clears memory with a memset, so a
forward + backward step can be captured once and replayed (a serving or
training loop that cannot afford a launch from the host per kernel).  Each
case captures its step, then three times: writes new logits into the
captured input buffers, poisons every output, replays the graph, and
compares every output and record bit for bit with an eager step on the same
inputs (eager work and a synchronisation sit between the replays).
"""

import pytest
import torch

from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _gen(seed, dev):
    return torch.Generator(device=dev).manual_seed(seed)


def _logp_case(dev, dtype, N, V, k, cap):
    g = _gen(11, dev)
    x = (torch.randn(N, V, generator=g, device=dev) * 3).to(dtype)
    t = torch.randint(0, V, (N, k), generator=g, device=dev)
    t[0, 0] = -100
    if k > 1:
        t[1, 1] = t[1, 0]
    gl = torch.randn(N, k, generator=g, device=dev)
    lp = torch.empty(N, k, dtype=torch.float32, device=dev)
    st = rlk.new_stats(rlk.RLK_HEAD_LOGP, N, V, dev)
    gx = torch.empty_like(x)

    def step():
        rlk.rlk_logp_fwd(x, t, cap, lp, st)
        rlk.rlk_logp_bwd(x, t, cap, st, gl, gx)

    return [x], [lp, st, gx], step


def _entropy_case(dev, dtype, N, V, cap):
    g = _gen(12, dev)
    x = (torch.randn(N, V, generator=g, device=dev) * 3).to(dtype)
    ge = torch.randn(N, generator=g, device=dev)
    h = torch.empty(N, dtype=torch.float32, device=dev)
    st = rlk.new_stats(rlk.RLK_HEAD_ENTROPY, N, V, dev)
    gx = torch.empty_like(x)

    def step():
        rlk.rlk_entropy_fwd(x, cap, h, st)
        rlk.rlk_entropy_bwd(x, cap, st, ge, gx)

    return [x], [h, st, gx], step


def _kl_case(dev, dtype, N, V, direction, cap):
    g = _gen(13, dev)
    x = (torch.randn(N, V, generator=g, device=dev) * 3).to(dtype)
    y = (x.float() + 0.5 * torch.randn(N, V, generator=g, device=dev)).to(dtype)
    gk = torch.randn(N, generator=g, device=dev)
    kl = torch.empty(N, dtype=torch.float32, device=dev)
    st = rlk.new_stats(rlk.RLK_HEAD_KL, N, V, dev)
    gx = torch.empty_like(x)
    gy = torch.empty_like(y)

    def step():
        rlk.rlk_kl_fwd(x, y, direction, cap, cap, kl, st)
        rlk.rlk_kl_bwd(x, y, direction, cap, cap, st, gk, gx)
        rlk.rlk_kl_bwd_ref(x, y, direction, cap, cap, st, gk, gy)

    return [x, y], [kl, st, gx, gy], step


def _softcap_case(dev):
    g = _gen(14, dev)
    x = (torch.randn(2, 3, 65536, generator=g, device=dev) * 40).to(torch.bfloat16)
    gy = torch.randn(2, 3, 65536, generator=g, device=dev)
    y = torch.empty(x.shape, dtype=torch.float32, device=dev)
    gx = torch.empty_like(x)

    def step():
        rlk.rlk_softcap_fwd(x, y, 20.0)
        rlk.rlk_softcap_bwd(x, gy, gx, 20.0)

    return [x], [y, gx], step


CASES = {
    "logp_fp32_k1": lambda d: _logp_case(d, torch.float32, 64, 32000, 1, 0.0),
    "logp_bf16_k4_cap30": lambda d: _logp_case(d, torch.bfloat16, 200, 32000, 4, 30.0),
    "logp_bf16_k64_cap20_wide": lambda d: _logp_case(d, torch.bfloat16, 96, 65536, 64, 20.0),
    "logp_f16_k300_topk": lambda d: _logp_case(d, torch.float16, 40, 20000, 300, 0.0),
    "entropy_bf16_cap30_table": lambda d: _entropy_case(d, torch.bfloat16, 1100, 65536, 30.0),
    "entropy_fp32": lambda d: _entropy_case(d, torch.float32, 100, 30011, 0.0),
    "kl_reverse_bf16": lambda d: _kl_case(d, torch.bfloat16, 128, 30016, 0, 0.0),
    "kl_forward_bf16_cap": lambda d: _kl_case(d, torch.bfloat16, 128, 30016, 1, 25.0),
    "softcap": _softcap_case,
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager_steps(dev, name):
    inputs, outputs, step = CASES[name](dev)
    originals = [t.clone() for t in inputs]
    # warm up on a side stream, then capture
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize(dev)
    for r in range(3):
        # new logits in the captured buffers: a permutation of the rows and,
        # on the second replay, a scaled copy
        for t, o in zip(inputs, originals):
            perm = torch.roll(torch.arange(o.shape[0], device=dev), r)
            t.copy_(o[perm] * (1.5 if r == 1 else 1.0))
        for o in outputs:
            o.view(torch.uint8).fill_(0xA5)
        graph.replay()
        torch.cuda.synchronize(dev)
        got = [_bits(o).clone() for o in outputs]
        for o in outputs:
            o.view(torch.uint8).fill_(0x5A)
        step()
        torch.cuda.synchronize(dev)
        for i, (a, o) in enumerate(zip(got, outputs)):
            ne = a != _bits(o)
            assert not bool(ne.any()), \
                f"{name}, replay {r}: output {i} differs bitwise in {int(ne.sum())} elements"
