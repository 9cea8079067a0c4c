"""Backward tail pieces of calls of at least 64 MiB, against the oracle.

Rows of whole 8-element chunks whose last piece is at least half full, in a
call of at least 64 MiB of logits, have that last piece computed by a launch
of its own (moved back to end at the row's end, storing only the columns the
full pieces did not).  Smaller calls take the ordinary tail path.  These
cases sit on the far side of that switch: V = 32000 (4000 chunks: 15 full
256-chunk pieces and a 160-chunk tail; 3 full 1024-chunk wide pieces and a
928-chunk tail, or, for k = 16, 7 full 512-chunk half-size wide pieces and
a 416-chunk tail) at 600 to 4200 rows.  Each case

  * asserts that the shape meets the switch's condition (a mirror of the
    rule the library applies, ``last_piece_apart``), so the test provably
    reaches the path;
  * compares at least 32 whole rows (the first, the last, every special row
    and seeded random rows) element by element with the fp64 oracle
    ("perf(logp): fused zero-workspace backward for the generic CUDA fused
    logp", RL-Kernel pull request 495, Tests: agreement with fp64 across V);
  * checks that a 4-row subset of the same rows, a call far below 64 MiB
    that takes the ordinary tail path, gives bit-identical outputs and
    gradients, and so does the subset at a misaligned base, which reads
    every element on its own and stores element by element (the same pull
    request's Summary: deterministic and batch-invariant).
"""

import numpy as np
import pytest
import torch

from tests.parity import assert_grad, assert_out, strict_bf16_misses, to64
from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu

V = 32000
PIECE_CHUNKS = 256    # one-shot piece: 256 lanes x 1 chunk (entropy, KL, logprobs k <= 4)
WIDE_CHUNKS = 1024    # wide piece: 256 lanes x 4 chunks (logprobs 4 < k <= 256)


def piece_chunks(k, V):
    """Chunks per backward piece for logprobs with k slots (the library's
    rule): one-shot pieces up to 4 slots; wide pieces above, half-size where
    a full wide piece would hold at most 5 targets on average."""
    if k <= 4:
        return PIECE_CHUNKS
    return WIDE_CHUNKS // 2 if k * WIDE_CHUNKS * 8 <= 5 * V else WIDE_CHUNKS


def last_piece_apart(N, V, esize, pc):
    """The library's switch (rlk_bwd_kernels.h, last_piece_apart), for
    16-byte aligned rows."""
    nfull = V // 8
    return (V % 8 == 0 and nfull >= pc and nfull // pc < 16 and 2 * (nfull % pc) >= pc
            and N * V * esize >= (64 << 20))


SHAPES = [(torch.bfloat16, 1100), (torch.float16, 1100), (torch.float32, 600),
          (torch.bfloat16, 4200)]   # the last one: write-through stores, streaming loads
SHAPE_IDS = ["bf16_1100", "f16_1100", "f32_600", "bf16_4200"]


def dgen(dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return g


def cgen(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def sample(N, special, n_random=30, seed=0):
    rnd = torch.randperm(N, generator=cgen(seed))[:n_random].tolist()
    return sorted(set(rnd) | {0, N - 1} | set(int(r) for r in special))


def check_subset_bits(full_out, full_gx, sub_out, sub_gx, rows, what):
    ri = torch.tensor(rows, device=full_gx.device)
    assert torch.equal(full_out[ri].view(torch.int32), sub_out.view(torch.int32)), \
        f"{what}: outputs of a row subset differ from the full call"
    a = full_gx[ri].contiguous().view(torch.int16 if full_gx.element_size() == 2 else torch.int32)
    b = sub_gx.contiguous().view(a.dtype)
    assert torch.equal(a, b), f"{what}: gradients of a row subset differ from the full call"


def misaligned(t):
    """A copy of t whose base is one element past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    m = buf[1:1 + t.numel()].view(t.shape)
    m.copy_(t)
    assert m.data_ptr() % 16 != 0
    return m


def logits(dev, dtype, N, std, seed):
    return (torch.randn(N, V, generator=dgen(dev, seed), device=dev) * std).to(dtype)


@pytest.mark.parametrize("k", [1, 4, 16, 64])
@pytest.mark.parametrize("cap", [0.0, 30.0])
@pytest.mark.parametrize("dtype,N", SHAPES, ids=SHAPE_IDS)
def test_logp_last_piece(dev, orc, dtype, N, k, cap):
    if N == 4200 and (k in (4, 16) or cap):
        pytest.skip("the 4200-row shape covers k = 1 and 64 without a cap")
    es = torch.tensor([], dtype=dtype).element_size()
    assert last_piece_apart(N, V, es, piece_chunks(k, V))
    x = logits(dev, dtype, N, 15.0 if cap else 3.0, 100 + k)
    x[7] += 1000.0
    t = torch.randint(0, V, (N, k), generator=cgen(k))
    gs = cgen(k + 1)
    for r in range(N):
        if k > 1:
            j, jj = torch.randint(0, k, (2,), generator=gs).tolist()
            t[r, j] = t[r, jj]                            # a duplicate id
    t[1, 0] = -100
    t[2, k - 1] = V + 7
    t[3] = -100                                           # fully ignored row
    # Targets on both sides of the cut of the moved-back last piece: it
    # recomputes chunks [nfull - pc, pc * (nfull // pc)) and stores from
    # chunk pc * (nfull // pc) on (wide pieces: columns 23808..24575 and
    # 24576..; half-size wide pieces 27904..28671 and 28672..; one-shot
    # pieces 29952..30719 and 30720..).
    t[5, 0] = V - 1
    t[6, 0] = 24575
    t[8, 0] = 24576
    t[9, 0] = 30719
    t[10, 0] = 30720
    t[11, 0] = 28671
    t[12, 0] = 28672
    g = torch.randn(N, k, generator=cgen(k + 2))
    td, gd = t.to(dev), g.to(dev)
    out, st = rlk.logp_fwd(x, td, cap)
    gx = rlk.logp_bwd(x, td, gd, st, cap)
    torch.cuda.synchronize()
    rows = sample(N, [1, 2, 3, 5, 6, 7, 8, 9, 10, 11, 12], seed=k)
    ri = torch.tensor(rows, device=dev)
    x64, t_np, g64 = to64(x[ri]), t[rows].numpy(), to64(g[rows])
    ref, refg = orc.logp_fwd(x64, t_np, cap), orc.logp_bwd(x64, t_np, g64, cap)
    ign = (t_np < 0) | (t_np >= V)
    assert_out(out[ri], ref, dtype, "logp", exact_zero=ign)
    assert_grad(gx[ri], refg, "logp grad", exact_zero=np.repeat(ign.all(1)[:, None], V, 1))
    if dtype == torch.bfloat16:
        print(f"logp k={k} cap={cap}: {strict_bf16_misses(gx[ri], refg)} elements beyond 4e-3")
    sub = [0, 3, 6, N - 1]
    si = torch.tensor(sub, device=dev)
    ts, gss = td[si].contiguous(), gd[si].contiguous()
    assert not last_piece_apart(len(sub), V, es, piece_chunks(k, V))
    for xs in (x[si].contiguous(), misaligned(x[si])):
        so, sst = rlk.logp_fwd(xs, ts, cap)
        sg = rlk.logp_bwd(xs, ts, gss, sst, cap)
        torch.cuda.synchronize()
        check_subset_bits(out, gx, so, sg, sub, f"logp k={k}, base % 16 = {xs.data_ptr() % 16}")


@pytest.mark.parametrize("cap", [0.0, 30.0])
@pytest.mark.parametrize("dtype,N", SHAPES, ids=SHAPE_IDS)
def test_entropy_last_piece(dev, orc, dtype, N, cap):
    es = torch.tensor([], dtype=dtype).element_size()
    assert last_piece_apart(N, V, es, PIECE_CHUNKS)
    x = logits(dev, dtype, N, 15.0 if cap else 3.0, 200)
    x[4] += 1000.0
    x[9] = 0.25                                           # uniform row
    if not cap:
        x[11] = float("-inf")                             # empty row
        x[12, V - 100:] = float("-inf")                   # masked tail columns
    g = torch.randn(N, generator=dgen(dev, 201), device=dev)
    H, st = rlk.entropy_fwd(x, cap)
    gx = rlk.entropy_bwd(x, g, st, cap)
    torch.cuda.synchronize()
    rows = sample(N, [4, 9, 11, 12], seed=5)
    ri = torch.tensor(rows, device=dev)
    x64 = to64(x[ri])
    assert_out(H[ri], orc.entropy_fwd(x64, cap), dtype, "entropy")
    masked = np.isneginf(x64) & ~np.isneginf(x64).all(1, keepdims=True) if not cap else None
    refg = orc.entropy_bwd(x64, to64(g[ri]), cap)
    assert_grad(gx[ri], refg, "entropy grad", exact_zero=masked)
    if dtype == torch.bfloat16:
        print(f"entropy cap={cap}: {strict_bf16_misses(gx[ri], refg)} elements beyond 4e-3")
    sub = [0, 11, 12, N - 1]
    si = torch.tensor(sub, device=dev)
    gs = g[si].contiguous()
    for xs in (x[si].contiguous(), misaligned(x[si])):
        sh, sst = rlk.entropy_fwd(xs, cap)
        sg = rlk.entropy_bwd(xs, gs, sst, cap)
        torch.cuda.synchronize()
        check_subset_bits(H, gx, sh, sg, sub, f"entropy, base % 16 = {xs.data_ptr() % 16}")


@pytest.mark.parametrize("direction", [0, 1], ids=["rev", "fwd"])
@pytest.mark.parametrize("cap", [0.0, 30.0])
@pytest.mark.parametrize("dtype,N", SHAPES[:3], ids=SHAPE_IDS[:3])
def test_kl_last_piece(dev, orc, dtype, N, cap, direction):
    es = torch.tensor([], dtype=dtype).element_size()
    assert last_piece_apart(N, V, es, PIECE_CHUNKS)
    a32 = torch.randn(N, V, generator=dgen(dev, 300), device=dev) * 3.0
    b32 = a32 + torch.randn(N, V, generator=dgen(dev, 301), device=dev) * 0.5
    special = [13]
    if not cap:
        b32[8, V - 3200:] = float("-inf")                 # support mismatch
        a32[10] = float("-inf")                           # empty in both
        b32[10] = float("-inf")
        special += [8, 10]
    a, b = a32.to(dtype), b32.to(dtype)
    del a32, b32
    g = torch.randn(N, generator=dgen(dev, 302), device=dev)
    D, st = rlk.kl_fwd(a, b, direction, cap, cap)
    gp = rlk.kl_bwd(a, b, g, st, direction, cap, cap)
    gr = rlk.kl_bwd_ref(a, b, g, st, direction, cap, cap)
    torch.cuda.synchronize()
    rows = sample(N, special, seed=6 + direction)
    ri = torch.tensor(rows, device=dev)
    a64, b64, g64 = to64(a[ri]), to64(b[ri]), to64(g[ri])
    assert_out(D[ri], orc.kl_fwd(a64, b64, direction, cap, cap), dtype, "kl")
    refp = orc.kl_bwd(a64, b64, g64, direction, cap, cap)
    assert_grad(gp[ri], refp, "kl grad (policy)")
    assert_grad(gr[ri], orc.kl_bwd_ref(a64, b64, g64, direction, cap, cap), "kl grad (ref)")
    if dtype == torch.bfloat16:
        print(f"kl dir={direction} cap={cap}: {strict_bf16_misses(gp[ri], refp)} elements "
              f"beyond 4e-3")
    sub = [0, 8, 10, N - 1]
    si = torch.tensor(sub, device=dev)
    sgv = g[si].contiguous()
    for sa, sb in ((a[si].contiguous(), b[si].contiguous()), (misaligned(a[si]), misaligned(b[si]))):
        sD, sst = rlk.kl_fwd(sa, sb, direction, cap, cap)
        sgp = rlk.kl_bwd(sa, sb, sgv, sst, direction, cap, cap)
        sgr = rlk.kl_bwd_ref(sa, sb, sgv, sst, direction, cap, cap)
        torch.cuda.synchronize()
        al = sa.data_ptr() % 16
        check_subset_bits(D, gp, sD, sgp, sub, f"kl policy, base % 16 = {al}")
        check_subset_bits(D, gr, sD, sgr, sub, f"kl reference, base % 16 = {al}")
