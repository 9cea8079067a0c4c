"""Seeded synthetic inputs for the five measured workloads (no method arithmetic).

This module only draws random tensors with the shapes, value distributions and
special structure (ignored targets, masked columns, offset rows, duplicate
top-k ids) of the workloads the pages time.  It holds none of the log-softmax
arithmetic and is shared by the tests, the benchmark and the smoke check.

Every tensor is a pure function of (workload, seed, device, row chunking):
``torch.Generator`` streams seeded from the workload seed, drawn in fixed row
chunks so that peak memory stays bounded for the 10 GB tensors.

Workloads (each takes its distribution from the page it stands in for; the
pages time random tensors: normal logits whose scale grows with the cap,
uniform targets, +1000 offset rows):
  c1_logp_fp32      logprobs k=1, fp32 [64, 32000] ~ N(0, 2^2), 4 rows -100
  c2_logp_bf16      logprobs k=1, bf16 [8192, 151936] ~ N(0, 3^2),
                    5% targets -100 and 0.1% targets V+7
  c3_kl_bf16        KL shard, bf16 [8192, 75968] x 2: policy ~ N(0, 3^2),
                    reference = policy + N(0, 0.5^2); 1% of rows have the last
                    10% of reference columns at -inf; one row all -inf (both)
  c4_entropy_cap30  entropy with cap 30, bf16 [32768, 151936] ~ N(0, 15^2),
                    64 rows offset by +1000 before bf16 rounding
  c5_topk_cap20     top-k logprobs (k=256) with cap 20, bf16 [2048, 262144]
                    ~ N(0, 10^2); 2% duplicate ids, 2% ids -100, one row fully
                    ignored; plus the standalone softcap on bf16 [2, 3, 262144]
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

IGNORE_INDEX = -100


@dataclass(frozen=True)
class Workload:
    name: str
    head: str                 # "logp" | "entropy" | "kl"
    N: int
    V: int
    dtype: torch.dtype
    std: float
    seed: int
    k: int = 1
    cap: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def esize(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()


WORKLOADS = {
    "c1_logp_fp32": Workload("c1_logp_fp32", "logp", 64, 32000, torch.float32, 2.0, 1,
                             extra={"ignored_rows": 4}),
    "c2_logp_bf16": Workload("c2_logp_bf16", "logp", 8192, 151936, torch.bfloat16, 3.0, 2,
                             extra={"ignored_frac": 0.05, "oob_frac": 0.001, "oob_offset": 7}),
    "c3_kl_bf16": Workload("c3_kl_bf16", "kl", 8192, 75968, torch.bfloat16, 3.0, 3,
                           extra={"ref_noise": 0.5, "mismatch_frac": 0.01, "mask_cols_frac": 0.1,
                                  "empty_rows": 1}),
    "c4_entropy_cap30": Workload("c4_entropy_cap30", "entropy", 32768, 151936, torch.bfloat16,
                                 15.0, 4, cap=30.0, extra={"offset_rows": 64, "offset": 1000.0}),
    "c5_topk_cap20": Workload("c5_topk_cap20", "logp", 2048, 262144, torch.bfloat16, 10.0, 5,
                              k=256, cap=20.0,
                              extra={"dup_frac": 0.02, "ignored_frac": 0.02, "ignored_rows": 1,
                                     "softcap_shape": (2, 3, 262144)}),
}

# Tensor ids keep the generator streams of different tensors apart.
_T_LOGITS, _T_REF, _T_TARGETS, _T_GRAD, _T_SELECT, _T_SOFTCAP = range(6)


def _gen(seed: int, tensor_id: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + tensor_id * 7919 + 17)
    return g


def normal_rows(N: int, V: int, std: float, dtype, seed: int, tensor_id: int, device,
                chunk_rows: int = 2048, offset_rows=None, offset: float = 0.0) -> torch.Tensor:
    """N(0, std^2) in fp32, rows in ``offset_rows`` shifted by ``offset``, cast to dtype."""
    out = torch.empty((N, V), dtype=dtype, device=device)
    g = _gen(seed, tensor_id, device)
    mark = None
    if offset_rows is not None and len(offset_rows):
        mark = torch.zeros(N, dtype=torch.bool, device=device)
        mark[offset_rows.to(device)] = True
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        z = torch.randn((r1 - r0, V), generator=g, device=device, dtype=torch.float32)
        z.mul_(std)
        if mark is not None:
            m = mark[r0:r1]
            if bool(m.any()):
                z[m] += offset
        out[r0:r1].copy_(z)
        del z
    return out


def row_selection(N: int, counts, seed: int, device="cpu"):
    """Disjoint sets of rows: the first counts[0] of a seeded permutation, then the next ..."""
    perm = torch.randperm(N, generator=_gen(seed, _T_SELECT, "cpu"))
    out, at = [], 0
    for c in counts:
        out.append(perm[at:at + c].sort().values.to(device))
        at += c
    return out


def frac_count(n: int, frac: float) -> int:
    return int(round(n * frac))


def make_inputs(name: str, device="cpu", N: int | None = None, V: int | None = None,
                with_grad: bool = True) -> dict:
    """Inputs of one workload.  ``N``/``V`` override the size (for small tests).

    Returns a dict with the logits (and reference for KL), int64 targets [N, k]
    for logprobs, fp32 upstream gradients, and the special-row index sets.
    """
    w = WORKLOADS[name]
    N = w.N if N is None else N
    V = w.V if V is None else V
    dev = torch.device(device)
    d: dict = {"workload": w, "N": N, "V": V}

    if w.head == "entropy":
        n_off = min(N, w.extra["offset_rows"])
        (off_rows,) = row_selection(N, [n_off], w.seed)
        d["offset_rows"] = off_rows
        d["logits"] = normal_rows(N, V, w.std, w.dtype, w.seed, _T_LOGITS, dev,
                                  offset_rows=off_rows, offset=w.extra["offset"])
    else:
        d["logits"] = normal_rows(N, V, w.std, w.dtype, w.seed, _T_LOGITS, dev)

    if w.head == "kl":
        n_mis = frac_count(N, w.extra["mismatch_frac"])
        n_emp = min(w.extra["empty_rows"], max(0, N - n_mis))
        mis_rows, empty_rows = row_selection(N, [n_mis, n_emp], w.seed)
        noise = normal_rows(N, V, w.extra["ref_noise"], torch.float32, w.seed, _T_REF, dev)
        ref = (d["logits"].float() + noise).to(w.dtype)
        del noise
        ncols = int(math.ceil(w.extra["mask_cols_frac"] * V))
        if n_mis:
            ref[mis_rows.to(dev), V - ncols:] = float("-inf")
        if n_emp:
            ref[empty_rows.to(dev)] = float("-inf")
            d["logits"][empty_rows.to(dev)] = float("-inf")
        d["ref"] = ref
        d["mismatch_rows"], d["empty_rows"] = mis_rows, empty_rows
        d["masked_cols"] = ncols

    if w.head == "logp":
        k = w.k
        gt = _gen(w.seed, _T_TARGETS, dev)
        t = torch.randint(0, V, (N, k), generator=gt, device=dev, dtype=torch.int64)
        if k == 1:
            if "ignored_frac" in w.extra:
                n_ign = frac_count(N, w.extra["ignored_frac"])
                n_oob = frac_count(N, w.extra["oob_frac"])
            else:
                n_ign, n_oob = min(N, w.extra["ignored_rows"]), 0
            ign_rows, oob_rows = row_selection(N, [n_ign, n_oob], w.seed)
            t[ign_rows.to(dev), 0] = IGNORE_INDEX
            if n_oob:
                t[oob_rows.to(dev), 0] = V + w.extra["oob_offset"]
            d["ignored_rows"], d["oob_rows"] = ign_rows, oob_rows
        else:
            n_slots = N * k
            n_dup = frac_count(n_slots, w.extra["dup_frac"])
            n_ign = frac_count(n_slots, w.extra["ignored_frac"])
            gsel = _gen(w.seed, _T_SELECT, "cpu")
            perm = torch.randperm(n_slots, generator=gsel)
            dup = perm[:n_dup].to(dev)
            ign = perm[n_dup:n_dup + n_ign].to(dev)
            # a duplicate copies the id of another slot of the same row
            shift = torch.randint(1, k, (n_dup,), generator=gsel).to(dev)
            rows, cols = dup // k, dup % k
            src = rows * k + (cols + shift) % k
            flat = t.view(-1)
            flat[dup] = flat[src].clone()
            flat[ign] = IGNORE_INDEX
            (full_rows,) = row_selection(N, [min(N, w.extra["ignored_rows"])], w.seed + 1)
            t[full_rows.to(dev)] = IGNORE_INDEX
            d["dup_slots"], d["ignored_slots"], d["ignored_rows"] = dup, ign, full_rows
        d["targets"] = t

    if with_grad:
        gg = _gen(w.seed, _T_GRAD, dev)
        gshape = (N, w.k) if w.head == "logp" else (N,)
        d["grad"] = torch.randn(gshape, generator=gg, device=dev, dtype=torch.float32)
    return d


def make_softcap_inputs(name: str = "c5_topk_cap20", device="cpu", shape=None, dtype=None):
    """Standalone softcap input x ~ N(0, std^2) and fp32 upstream gradient."""
    w = WORKLOADS[name]
    shape = tuple(shape or w.extra["softcap_shape"])
    dtype = dtype or w.dtype
    g = _gen(w.seed, _T_SOFTCAP, torch.device(device))
    x = (torch.randn(shape, generator=g, device=device) * w.std).to(dtype)
    gy = torch.randn(shape, generator=g, device=device)
    return x, gy
