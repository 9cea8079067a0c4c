"""Determinism and invariance of the HIP path (bitwise, no tolerance).

The claims ("L0 repeatable, L1 batch-invariant" in the vocabulary of RL-Kernel
pull request 507):
  * repeat: the same call twice gives identical bits;
  * batch invariance: a row's outputs and gradient do not depend on which
    other rows are in the batch, on their order, or on N;
  * layout invariance: a padded row stride (ld > V, padding filled with NaN,
    so any stray read shows up; the technique of the strided-view test in
    DeepSpeed pull request 8838) and a misaligned base pointer give the same
    bits as the contiguous aligned call;
  * dtype: a bf16 tensor and the fp32 tensor holding the same values give
    identical head outputs, and the bf16 gradient is the round-to-nearest-even
    of the fp32 one (the side effect reported on the same pull request).
"""

import pytest
import torch

from vocab_log_softmax_amd import rlk

pytestmark = pytest.mark.gpu


def _gen(seed):
    return torch.Generator().manual_seed(seed)


def run_all(x, ref, t, g_t, g_r, cap):
    """Outputs and gradients of every head for logits x (and ref for KL)."""
    out = {}
    lp, st = rlk.logp_fwd(x, t, cap)
    out["logp"] = lp
    out["logp_grad"] = rlk.logp_bwd(x, t, g_t, st, cap)
    h, st = rlk.entropy_fwd(x, cap)
    out["ent"] = h
    out["ent_grad"] = rlk.entropy_bwd(x, g_r, st, cap)
    for d in (0, 1):
        k, st = rlk.kl_fwd(x, ref, d, cap, 0.0)
        out[f"kl{d}"] = k
        out[f"kl{d}_grad"] = rlk.kl_bwd(x, ref, g_r, st, d, cap, 0.0)
    torch.cuda.synchronize()
    return out


def make(N, V, dtype, seed, dev, k=3):
    x = (torch.randn(N, V, generator=_gen(seed)) * 4).to(dtype)
    ref = (x.float() + torch.randn(N, V, generator=_gen(seed + 1)) * 0.5).to(dtype)
    x[1, : V // 3] = float("-inf")
    ref[1, : V // 3] = float("-inf")
    t = torch.randint(0, V, (N, k), generator=_gen(seed + 2))
    t[0, 1] = -100
    g_t = torch.randn(N, k, generator=_gen(seed + 3))
    g_r = torch.randn(N, generator=_gen(seed + 4))
    return [a.to(dev) for a in (x, ref, t, g_t, g_r)]


def assert_bitwise(a, b, what):
    assert a.shape == b.shape and a.dtype == b.dtype, what
    ai = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
    bi = b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
    ne = (ai != bi)
    assert not bool(ne.any()), f"{what}: {int(ne.sum())} elements differ bitwise"


@pytest.mark.parametrize("V", [1031, 32000, 151936])
@pytest.mark.parametrize("cap", [0.0, 30.0, 50.0])
def test_repeat_is_bitwise(dev, V, cap):
    args = make(16, V, torch.bfloat16, V, dev)
    a = run_all(*args, cap)
    b = run_all(*args, cap)
    for k in a:
        assert_bitwise(a[k], b[k], f"repeat {k}")


@pytest.mark.parametrize("V", [4097, 151936])
def test_batch_invariance(dev, V):
    N = 40
    x, ref, t, g_t, g_r = make(N, V, torch.bfloat16, 7, dev)
    full = run_all(x, ref, t, g_t, g_r, 20.0)
    perm = torch.randperm(N, generator=_gen(1)).to(dev)
    shuf = run_all(x[perm].contiguous(), ref[perm].contiguous(), t[perm].contiguous(),
                   g_t[perm].contiguous(), g_r[perm].contiguous(), 20.0)
    sub = torch.tensor([3, 17, 1, 39], device=dev)
    part = run_all(x[sub].contiguous(), ref[sub].contiguous(), t[sub].contiguous(),
                   g_t[sub].contiguous(), g_r[sub].contiguous(), 20.0)
    single = run_all(x[5:6].contiguous(), ref[5:6].contiguous(), t[5:6].contiguous(),
                     g_t[5:6].contiguous(), g_r[5:6].contiguous(), 20.0)
    for k in full:
        assert_bitwise(full[k][perm], shuf[k], f"permuted {k}")
        assert_bitwise(full[k][sub], part[k], f"subset {k}")
        assert_bitwise(full[k][5:6], single[k], f"single row {k}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16],
                         ids=["f32", "bf16", "f16"])
def test_batch_invariance_across_load_policy(dev, dtype):
    # Operands above 256 MiB are read with non-temporal loads, smaller ones
    # with ordinary loads; the rows of a large batch and of a small subset of
    # it must still agree bit for bit.
    N, V = 1100, 131072                    # 288 MB per tensor in 16 bits
    g = torch.Generator(device=dev).manual_seed(11)
    x = (torch.randn(N, V, generator=g, device=dev) * 4).to(dtype)
    ref = (x.float() + torch.randn(N, V, generator=g, device=dev) * 0.5).to(dtype)
    t = torch.randint(0, V, (N, 3), generator=g, device=dev)
    g_t = torch.randn(N, 3, generator=g, device=dev)
    g_r = torch.randn(N, generator=g, device=dev)
    sub = torch.arange(0, N, 17, device=dev)  # 65 rows: 17 MB in 16 bits
    for cap in (0.0, 30.0):
        full = run_all(x, ref, t, g_t, g_r, cap)
        part = run_all(x[sub].contiguous(), ref[sub].contiguous(), t[sub].contiguous(),
                       g_t[sub].contiguous(), g_r[sub].contiguous(), cap)
        for k in full:
            assert_bitwise(full[k][sub], part[k], f"cap {cap} {k}")
        del full, part


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_cap_table_and_computed_odd_form_agree(dev, dtype):
    # Under the fixed cap, long rows of 16-bit logits read their statistic
    # inputs from an LDS table once a call has 1024 rows or more and compute
    # them below that; fp32 logits always compute them.  Rows wide enough for
    # the odd form in both heads (logprobs from 196608 columns), a call of
    # 1030 rows (table kernel, aligned and misaligned), a 65-row subset and
    # its fp32 copy (computed) must agree bit for bit, record and gradient
    # included.
    N, V = 1030, 196616
    g = torch.Generator(device=dev).manual_seed(23)
    x = (torch.randn(N, V, generator=g, device=dev) * 4).to(dtype)
    x[3, :1000] = float("inf")
    x[4, 5:9] = float("-inf")
    t = torch.randint(0, V, (N, 3), generator=g, device=dev)
    g_t = torch.randn(N, 3, generator=g, device=dev)
    g_r = torch.randn(N, generator=g, device=dev)
    sub = torch.arange(0, N, 16, device=dev)
    buf = torch.empty(N * V + 1, dtype=dtype, device=dev)
    xm = buf[1:].view(N, V)
    xm.copy_(x)
    cap = 20.0

    def heads(xx, tt, gt, gr):
        lp, st = rlk.logp_fwd(xx, tt, cap)
        h, sh = rlk.entropy_fwd(xx, cap)
        n = xx.shape[0]
        out = {"logp": lp, "logp_rec": st.view(n, -1), "ent": h, "ent_rec": sh.view(n, -1),
               "logp_grad": rlk.logp_bwd(xx, tt, gt, st, cap),
               "ent_grad": rlk.entropy_bwd(xx, gr, sh, cap)}
        torch.cuda.synchronize()
        return out

    full = heads(x, t, g_t, g_r)
    mis = heads(xm, t, g_t, g_r)
    for k in full:
        assert_bitwise(mis[k], full[k], f"misaligned {k}")
    del mis
    part = heads(x[sub].contiguous(), t[sub].contiguous(), g_t[sub].contiguous(),
                 g_r[sub].contiguous())
    wide = heads(x[sub].float(), t[sub].contiguous(), g_t[sub].contiguous(),
                 g_r[sub].contiguous())
    for k in full:
        assert_bitwise(full[k][sub], part[k], f"subset {k}")
        if k.endswith("grad"):
            assert_bitwise(part[k], wide[k].to(dtype), f"fp32 copy {k}")
        else:
            assert_bitwise(part[k], wide[k], f"fp32 copy {k}")
    assert torch.isfinite(full["logp"][:5]).all() and torch.isfinite(full["ent"][:5]).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16],
                         ids=["f32", "bf16", "f16"])
@pytest.mark.parametrize("V,pad", [(4096, 8), (4099, 5), (151936, 64)])
def test_padded_stride_reads_nothing_outside_the_row(dev, dtype, V, pad):
    N = 12
    x, ref, t, g_t, g_r = make(N, V, dtype, V + pad, dev)
    want = run_all(x, ref, t, g_t, g_r, 0.0)
    xp = torch.full((N, V + pad), float("nan"), dtype=dtype, device=dev)
    rp = torch.full((N, V + pad), float("nan"), dtype=dtype, device=dev)
    xp[:, :V] = x
    rp[:, :V] = ref
    got = run_all(xp[:, :V], rp[:, :V], t, g_t, g_r, 0.0)
    for k in want:
        assert_bitwise(want[k], got[k], f"padded {k}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_misaligned_base_pointer(dev, dtype):
    N, V = 9, 8192
    x, ref, t, g_t, g_r = make(N, V, dtype, 99, dev)
    want = run_all(x, ref, t, g_t, g_r, 30.0)
    bx = torch.empty(N * V + 1, dtype=dtype, device=dev)
    br = torch.empty(N * V + 1, dtype=dtype, device=dev)
    xs = bx[1:].view(N, V)
    rs = br[1:].view(N, V)
    xs.copy_(x)
    rs.copy_(ref)
    assert xs.data_ptr() % 16 != 0
    got = run_all(xs, rs, t, g_t, g_r, 30.0)
    for k in want:
        assert_bitwise(want[k], got[k], f"misaligned {k}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("cap", [0.0, 20.0, 60.0])
def test_half_dtypes_equal_fp32_of_same_values(dev, dtype, cap):
    N, V = 10, 75968
    x, ref, t, g_t, g_r = make(N, V, dtype, 5, dev)
    b = run_all(x, ref, t, g_t, g_r, cap)
    f = run_all(x.float(), ref.float(), t, g_t, g_r, cap)
    for k in b:
        if k.endswith("grad"):
            assert_bitwise(b[k], f[k].to(dtype), f"{dtype} grad == RNE(fp32 grad) {k}")
        else:
            assert_bitwise(b[k], f[k], f"{dtype} vs fp32 output {k}")


def _layout_targets(N, V, k, seed):
    """Target ids on the edges of the backward's lane layouts: for the lane
    t of a 2048-column slot (one 256-lane chunk slot), the last column of its
    first four and the first of its next four (16-bit: one chunk; fp32 full
    pieces: quads t and 256 + t, 1024 columns apart), slot and piece
    boundaries, duplicates, the row's tail and, for k > 4, uniform fill."""
    g = _gen(seed)
    t = torch.randint(0, V, (N, k), generator=g)
    full = V // 2048 * 2048
    for r in range(N):
        lane = (37 * r) % 256
        slot = r % (full // 2048)
        base = slot * 2048
        edge = [base + 4 * lane + 3, base + 1024 + 4 * lane, base + 4 * lane + 4,
                base + 1024 + 4 * lane + 3, base + 2047, base, full + (r % (V - full))]
        for j in range(min(k, len(edge))):
            t[r, j] = edge[j]
        if k >= 4:
            t[r, k - 1] = t[r, 0]  # duplicate
    if k > 8:
        t[:, k // 2: k // 2 + k // 8] = t[:, : k // 8]
    t[::7, 1] = -100
    return t


@pytest.mark.parametrize("k,N", [(4, 300), (8, 300), (16, 300), (256, 300), (300, 300),
                                 (300, 600)])
@pytest.mark.parametrize("cap", [0.0, 20.0])
def test_fp32_piece_layout_matches_bf16(dev, k, N, cap):
    # fp32 full backward pieces hold two 16-byte quads 1024 columns apart per
    # lane and chunk slot, and fp32 row walks load and store each chunk's
    # halves through a lane swap; 16-bit ones hold one chunk.  The bf16
    # gradient must still be the round-to-nearest-even of the fp32 one at
    # every column, target columns included (k = 4: one-shot pieces; 8:
    # half-size wide pieces; 16 and 256: wide pieces, whose slot lists are
    # scanned, or sorted when a piece holds more than 16; 300: the top-k row kernel, in column segments for
    # 300 rows and one workgroup per row for 600).
    V = 16680
    x = (torch.randn(N, V, generator=_gen(71)) * (10.0 if cap else 3.0)).to(torch.bfloat16)
    t = _layout_targets(N, V, k, 72 + k)
    g_t = torch.randn(N, k, generator=_gen(73))
    x, t, g_t = x.to(dev), t.to(dev), g_t.to(dev)
    lp_b, st_b = rlk.logp_fwd(x, t, cap)
    gx_b = rlk.logp_bwd(x, t, g_t, st_b, cap)
    xf = x.float()
    lp_f, st_f = rlk.logp_fwd(xf, t, cap)
    gx_f = rlk.logp_bwd(xf, t, g_t, st_f, cap)
    torch.cuda.synchronize()
    assert_bitwise(lp_b, lp_f, f"logp k={k}")
    assert_bitwise(gx_b, gx_f.to(torch.bfloat16), f"grad k={k}")


def test_outputs_independent_of_stats_buffer_history(dev):
    # the forward record is fully rewritten: garbage in the buffer changes nothing
    x, ref, t, g_t, g_r = make(6, 5000, torch.bfloat16, 3, dev)
    lp, st = rlk.logp_fwd(x, t)
    g1 = rlk.logp_bwd(x, t, g_t, st)
    st2 = torch.full_like(st, 0xAB)
    out2 = torch.empty_like(lp)
    rlk.rlk_logp_fwd(x, t, 0.0, out2, st2)
    g2 = rlk.logp_bwd(x, t, g_t, st2)
    torch.cuda.synchronize()
    assert_bitwise(lp, out2, "logp")
    assert_bitwise(g1, g2, "grad")


@pytest.mark.parametrize("N", [37, 700])
@pytest.mark.parametrize("cap", [0.0, 20.0, 60.0])
def test_piece_and_wide_backward_kernels_agree(dev, N, cap):
    # k <= 4 runs the one-shot piece kernel, k = 5 the wide top-k piece
    # kernel; a fifth slot that is ignored changes neither G nor any one-hot
    # sum, so both must give the same bits.
    V = 9001
    x = (torch.randn(N, V, generator=_gen(11)) * 3).to(torch.bfloat16).to(dev)
    t4 = torch.randint(0, V, (N, 4), generator=_gen(12))
    t4[::7, 2] = t4[::7, 0]          # duplicates
    t4[::5, 1] = -100                # ignored
    t5 = torch.cat([t4, torch.full((N, 1), -100, dtype=torch.int64)], 1)
    g4 = torch.randn(N, 4, generator=_gen(13))
    g5 = torch.cat([g4, torch.randn(N, 1, generator=_gen(14))], 1)
    t4, t5, g4, g5 = t4.to(dev), t5.to(dev), g4.to(dev), g5.to(dev)
    lp4, st4 = rlk.logp_fwd(x, t4, cap)
    lp5, st5 = rlk.logp_fwd(x, t5, cap)
    gx4 = rlk.logp_bwd(x, t4, g4, st4, cap)
    gx5 = rlk.logp_bwd(x, t5, g5, st5, cap)
    torch.cuda.synchronize()
    assert_bitwise(lp4, lp5[:, :4], "forward outputs")
    assert_bitwise(gx4, gx5, "gradients of the two backward kernels")


@pytest.mark.parametrize("N", [37, 700])
@pytest.mark.parametrize("cap", [0.0, 20.0, 60.0])
def test_wide_and_topk_backward_kernels_agree(dev, N, cap):
    # k = 256 runs the wide top-k piece kernel, k = 257 the top-k row kernel
    # (37 rows: column segments; 700 rows: one workgroup per row); the extra
    # slot is ignored, so both must give the same bits.  Rows with heavy
    # duplication, an all-ignored row and (without the cap) an empty row.
    V = 20011
    x = (torch.randn(N, V, generator=_gen(21)) * 4).to(torch.bfloat16)
    if not cap:
        x[3] = float("-inf")
    t = torch.randint(0, V, (N, 256), generator=_gen(22))
    t[:, 100:140] = t[:, 60:100]      # duplicates within the row
    t[::3, 7] = t[::3, 0]
    t[1, :] = torch.randint(0, 40, (256,), generator=_gen(23))  # few columns, many repeats
    t[2, :] = -100                    # no valid slot
    t[::5, 200:210] = -100
    t[4, 255] = V + 3                 # out of range
    g = torch.randn(N, 256, generator=_gen(24))
    t7 = torch.cat([t, torch.full((N, 1), -100, dtype=torch.int64)], 1)
    g7 = torch.cat([g, torch.randn(N, 1, generator=_gen(25))], 1)
    x, t, t7, g, g7 = x.to(dev), t.to(dev), t7.to(dev), g.to(dev), g7.to(dev)
    lp, st = rlk.logp_fwd(x, t, cap)
    lp7, st7 = rlk.logp_fwd(x, t7, cap)
    gx = rlk.logp_bwd(x, t, g, st, cap)
    gx7 = rlk.logp_bwd(x, t7, g7, st7, cap)
    torch.cuda.synchronize()
    assert_bitwise(lp, lp7[:, :256], "forward outputs")
    assert_bitwise(gx, gx7, "gradients of the two backward kernels")
