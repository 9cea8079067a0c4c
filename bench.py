#!/usr/bin/env python3
"""Benchmark: fused logprobs forward + backward on one MI355X.

A step is one forward + backward pass of the hot path over one batch: the
single-read row statistics with the target gather (rlk_logp_fwd), then the
fused zero-workspace backward (rlk_logp_bwd), on the logprobs k=1 workload
bf16 logits [8192, 151936] (seeded synthetic inputs, already resident in HBM).

Prints ONE JSON line with the throughput in algorithmic GB/s (every logit
read once by the forward, read once and written once by the backward, plus the
per-row side arrays), the dominant kernel's roofline figures measured with HIP
events on the launch stream, and the fp64 CPU oracle timed on a bounded sample
of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
METRIC = "fwd+bwd ms and HBM GB/s (% of 8 TB/s) for logp/entropy/KL at N x V"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "vocab_log_softmax_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, kernel: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None.

    The summary must name the same kernel sources (hash) as this tree; a
    changed kernel makes its counters stale.
    """
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"^source_hash:\s*(\S+)", txt, re.M)
    m_rd = re.search(r"^hbm_read_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    m_wr = re.search(r"^hbm_write_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not (m_hash and m_rd and m_wr) or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_rd.group(1)) + float(m_wr.group(1))


class HipEvents:
    """Raw hipEvent_t timers, recorded on a raw stream handle.

    torch.cuda.Event.record costs a few microseconds of host time per call,
    which would dominate a launch-bound workload's step; hipEventRecord on
    the HIP runtime torch already loaded costs a fraction of that.  The
    events only time: they are read after a full device synchronisation, so
    they are created without the system-scope fence a default event record
    performs (its cache writeback and invalidation would slow the kernels
    that follow each marker).
    """

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, n: int, torch):
        lib_dir = os.path.join(os.path.dirname(torch.__file__), "lib")
        path = os.path.join(lib_dir, "libamdhip64.so")
        # same soname as the runtime torch loaded -> the same instance
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")
        self.ev = [ctypes.c_void_p() for _ in range(n)]
        for e in self.ev:
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e),
                                                ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, i: int, stream) -> None:
        self.hip.hipEventRecord(self.ev[i], stream)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self) -> None:
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def measure_ceilings(w, dev, torch) -> dict:
    """Practical HBM ceilings at the workload's tensor size (libceiling.so).

    Read-only, write-only and copy streams of 16-byte nontemporal accesses,
    grid-stride and row by row (one workgroup per row of V logits, as the
    library's kernels stream); median of 15 timed launches after 3 warm-up
    launches, HIP events on the current stream.
    """
    from vocab_log_softmax_amd import build as B

    if not os.path.exists(B.CEILING_LIB):
        raise SystemExit(f"{B.CEILING_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(B.CEILING_LIB)
    lib.ceiling_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.ceiling_run.restype = ctypes.c_int
    row_bytes = w.V * w.esize
    bytes_ = w.N * row_bytes
    src = torch.ones(bytes_ // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    raw = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ev = HipEvents(2 * 15, torch)
    out = {"bytes_per_tensor": bytes_, "row_bytes": row_bytes}
    kinds = {"read_grid_stride": (0, 1), "write_grid_stride": (1, 1), "copy_grid_stride": (2, 2),
             "read_rows": (3, 1), "copy_rows": (4, 2)}
    for name, (kind, passes) in kinds.items():
        def run():
            rc = lib.ceiling_run(kind, src.data_ptr(), dst.data_ptr(), bytes_, row_bytes,
                                 sink.data_ptr(), raw)
            if rc != 0:
                raise RuntimeError(f"ceiling_run({name}) failed: {rc}")
        for _ in range(3):
            run()
        for i in range(15):
            ev.record(2 * i, raw)
            run()
            ev.record(2 * i + 1, raw)
        torch.cuda.synchronize()
        ts = sorted(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(15))
        ms = ts[len(ts) // 2]
        out[name] = {"ms": round(ms, 4), "GB/s": round(passes * bytes_ / (ms * 1e-3) / 1e9, 1)}
    ev.close()
    return {"ceilings": out, "workload": w.name}


def time_softcap(name: str, dev, torch, reps: int = 50) -> dict:
    """The standalone softcap forward (y fp32) and backward on the workload's
    softcap tensor: mean kernel time over `reps` launches, HIP events."""
    from vocab_log_softmax_amd import rlk, workloads

    w = workloads.WORKLOADS[name]
    x, gy = workloads.make_softcap_inputs(name, dev)
    y = torch.empty(x.shape, dtype=torch.float32, device=dev)
    gx = torch.empty_like(x)
    n, es = x.numel(), x.element_size()
    raw = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    out = {"shape": list(x.shape), "dtype": str(x.dtype).replace("torch.", ""), "cap": w.cap}
    for what, fn, nbytes in (("fwd", lambda: rlk.rlk_softcap_fwd(x, y, w.cap), n * (es + 4)),
                             ("bwd", lambda: rlk.rlk_softcap_bwd(x, gy, gx, w.cap),
                              n * (es + 4 + es))):
        for _ in range(5):
            fn()
        ev = HipEvents(2, torch)
        torch.cuda.synchronize()
        ev.record(0, raw)
        for _ in range(reps):
            fn()
        ev.record(1, raw)
        torch.cuda.synchronize()
        ms = ev.elapsed_ms(0, 1) / reps
        ev.close()
        out[what] = {"us": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "bytes": nbytes}
    return out


def fwd1_name(w, N, V, es):
    """Which single-tensor forward kernel the library launches for this call.

    Mirrors the dispatch rule: under the fixed-form cap (2 c log2 e within
    [2^-16, 120]), rows of at least 65536 columns (entropy) or 196608
    (logprobs) take the odd form, read from the LDS table for 16-bit logits
    once the call has 1024 rows; only the kernel's name is taken from here.
    """
    sc = 2.0 * w.cap / math.log(2.0) if w.cap > 0 else 0.0
    fixed = 2.0 ** -16 <= sc <= 120.0
    min_cols = 65536 if w.head == "entropy" else 196608
    if fixed and es == 2 and V >= min_cols and N >= 1024:
        return "fwd1_tab_kernel"
    return "fwd1_kernel"


def side_bytes(w, N):
    """Per-step bytes of the per-row side arrays (targets, grads, outputs, stats)."""
    k = w.k
    if w.head == "logp":
        fwd = N * (8 * k + 4 * k + 32)
        bwd = N * (8 * k + 4 * k + 32)
    else:
        fwd = N * (4 + 32)
        bwd = N * (4 + 32)
    return fwd, bwd


def run_oracle_sample(w, d, max_rows: int, threads: int, min_seconds: float = 1.0,
                      direction: int = 0):
    """Time the fp64 oracle's fwd+bwd on the first max_rows rows (host cores).

    A sample that takes less than min_seconds is repeated (up to 1000 times)
    and the mean time of one pass is returned with the pass count.
    """
    import oracle

    orc = oracle.get()
    orc.set_threads(threads)
    n = min(max_rows, d["N"])
    x = d["logits"][:n].double().cpu().numpy()
    g = d["grad"][:n].double().cpu().numpy()
    t = d["targets"][:n].cpu().numpy() if w.head == "logp" else None
    r = d["ref"][:n].double().cpu().numpy() if w.head == "kl" else None

    def one_pass():
        if w.head == "logp":
            orc.logp_fwd(x, t, w.cap)
            orc.logp_bwd(x, t, g, w.cap)
        elif w.head == "entropy":
            orc.entropy_fwd(x, w.cap)
            orc.entropy_bwd(x, g, w.cap)
        else:
            orc.kl_fwd(x, r, direction, 0.0, 0.0)
            orc.kl_bwd(x, r, g, direction, 0.0, 0.0)

    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 1000:
            break
    return n, dt / passes, passes


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: at least 50, enough for 0.2 s of work)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: at least 5, enough for 50 ms)")
    ap.add_argument("--workload", default="c2_logp_bf16")
    ap.add_argument("--oracle-rows", type=int, default=8192,
                    help="rows of the workload timed on the CPU oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-threads", type=int, default=None,
                    help="host threads of the CPU oracle (default: the process's cores, "
                         "at most 16)")
    ap.add_argument("--rows", type=int, default=None,
                    help="override the workload's row count N (same recipe, e.g. 32768 rows "
                         "of c2_logp_bf16 for the pages' B200 comparison)")
    ap.add_argument("--direction", type=int, default=0, choices=(0, 1),
                    help="KL workloads: 0 reverse KL(policy||ref), 1 forward KL(ref||policy)")
    ap.add_argument("--cold", action="store_true",
                    help="write a 1 GiB buffer before every step (flushes the 256 MB Infinity "
                         "Cache and the L2s) and time the two kernels with events only")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the read / write / copy ceilings at the workload's size")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of a known size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(rows shard across GPUs with no exchange; vocabulary shards need one "
              "all-gather of the rlk_*_fwd_partial records before rlk_combine). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from vocab_log_softmax_amd import rlk, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    rlk.load_library()
    dev = torch.device("cuda:0")
    if args.copy_probe:
        # A plain copy of exactly 2 GiB each way: the HBM counters of this
        # kernel (2 GiB read, 2 GiB written per launch) calibrate FETCH_SIZE
        # and WRITE_SIZE for the traffic field.
        src = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": src.numel(), "launches": 3}))
        return 0
    w = workloads.WORKLOADS[args.workload]
    if args.ceilings:
        print(json.dumps(measure_ceilings(w, dev, torch)))
        return 0
    d = workloads.make_inputs(args.workload, dev, N=args.rows)
    x = d["logits"]
    N, V = x.shape
    es = x.element_size()
    stream = torch.cuda.current_stream(dev)

    if w.head == "logp":
        tg, g = d["targets"], d["grad"]
        out = torch.empty(tg.shape, dtype=torch.float32, device=dev)
        st = rlk.new_stats(rlk.RLK_HEAD_LOGP, N, V, dev)
        gx = torch.empty_like(x)
        fwd = rlk.prepare(rlk.rlk_logp_fwd, x, tg, w.cap, out, st)
        bwd = rlk.prepare(rlk.rlk_logp_bwd, x, tg, w.cap, st, g, gx)
        # k <= 4 slots: one-shot pieces; up to 256: wide pieces; wider: the row kernel
        n_in, fwd_name = 1, fwd1_name(w, N, V, es)
        bwd_name = ("bwd_piece_kernel" if w.k <= 4 else
                    "bwd_wide_kernel" if w.k <= 256 else "bwd_topk_kernel")
    elif w.head == "entropy":
        g = d["grad"]
        out = torch.empty(N, dtype=torch.float32, device=dev)
        st = rlk.new_stats(rlk.RLK_HEAD_ENTROPY, N, V, dev)
        gx = torch.empty_like(x)
        fwd = rlk.prepare(rlk.rlk_entropy_fwd, x, w.cap, out, st)
        bwd = rlk.prepare(rlk.rlk_entropy_bwd, x, w.cap, st, g, gx)
        n_in, fwd_name, bwd_name = 1, fwd1_name(w, N, V, es), "bwd_piece_kernel"
    else:
        ref, g = d["ref"], d["grad"]
        out = torch.empty(N, dtype=torch.float32, device=dev)
        st = rlk.new_stats(rlk.RLK_HEAD_KL, N, V, dev)
        gx = torch.empty_like(x)
        kd = args.direction
        fwd = rlk.prepare(rlk.rlk_kl_fwd, x, ref, kd, 0.0, 0.0, out, st)
        bwd = rlk.prepare(rlk.rlk_kl_bwd, x, ref, kd, 0.0, 0.0, st, g, gx)
        n_in, fwd_name, bwd_name = 2, "fwdkl_kernel", "bwd_piece_kernel"

    sf, sb = side_bytes(w, N)
    fwd_bytes = n_in * N * V * es + sf            # read every input logit once
    bwd_bytes = (n_in + 1) * N * V * es + sb      # read again, write the gradient once
    step_bytes = fwd_bytes + bwd_bytes

    # Warm-up.  Without --warmup / --steps both are sized from the step time:
    # a launch-bound step (microseconds) needs thousands of steps before clocks
    # and queues settle and for the timed region to outweigh its start-up.
    def run(n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fwd()
            bwd()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / max(1, n)

    if args.warmup is not None:
        warm_ms = run(args.warmup)
    else:
        run(5)                   # first launches (code loading, clocks)
        warm_ms = run(10)        # the step time, from settled launches
        extra = max(0, math.ceil(50.0 / max(warm_ms, 1e-6)) - 15)
        run(extra)
        args.warmup = 15 + extra
    if args.steps is None:
        args.steps = max(50, math.ceil(200.0 / max(warm_ms, 1e-6)))

    # HIP events on the stream the kernels run on, three per sampled step:
    # before the forward, between forward and backward, after the backward.
    # Every step is sampled unless a step is so short (launch-bound) that the
    # event markers themselves would show in its wall time; then every
    # tenth step is.
    stride = 1 if (warm_ms > 0.2 or args.cold) else 10
    sampled = list(range(0, args.steps, stride))
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.cold else None
    ev = HipEvents(3 * len(sampled), torch)
    raw = ctypes.c_void_p(stream.cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    j = 0
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(float(i))
        if i % stride == 0:
            ev.record(3 * j, raw)
            fwd()
            ev.record(3 * j + 1, raw)
            bwd()
            ev.record(3 * j + 2, raw)
            j += 1
        else:
            fwd()
            bwd()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = sum(ev.elapsed_ms(3 * j, 3 * j + 1) for j in range(len(sampled))) / len(sampled)
    bwd_ms = sum(ev.elapsed_ms(3 * j + 1, 3 * j + 2) for j in range(len(sampled))) / len(sampled)
    ev.close()
    ms_per_step = wall * 1e3 / args.steps
    if args.cold:  # the flush is not part of a step: the kernels' event time
        ms_per_step = fwd_ms + bwd_ms
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    bwd_gbs = bwd_bytes / (bwd_ms * 1e-3) / 1e9
    fwd_gbs = fwd_bytes / (fwd_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(args.workload, bwd_name)
    roofline = {
        "bound": "hbm",
        "kernel": f"{bwd_name} ({w.head} backward)",
        "achieved": round(bwd_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(bwd_gbs / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": bwd_bytes,
        "avg_launch_ms": round(bwd_ms, 4),
        "event_timed_steps": len(sampled),
        "second_kernel": {"kernel": f"{fwd_name} ({w.head} forward)", "avg_launch_ms":
                          round(fwd_ms, 4), "achieved": round(fwd_gbs, 1),
                          "frac": round(fwd_gbs / HBM_PEAK_GBS, 4),
                          "algorithmic_bytes_per_launch": fwd_bytes},
    }

    cpu = None
    if not args.no_cpu_baseline:
        threads = args.oracle_threads or min(len(os.sched_getaffinity(0)), 16)
        n, dt, passes = run_oracle_sample(w, d, args.oracle_rows, threads,
                                          direction=args.direction)
        sample_bytes = step_bytes * n / N
        cpu = {"value": round(sample_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"fp64 oracle fwd+bwd on the first {n} of {N} rows of the same "
                         f"workload ({n * V} logits per tensor), {dt:.3f} s wall per pass, "
                         f"mean of {passes} pass{'es' if passes > 1 else ''}"}

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "timing": ("cold: 1 GiB written before every step, step = forward + backward event time"
                   if args.cold else "warm: back-to-back steps, wall clock"),
        "config": {
            "workload": f"{args.workload}" + (f" (N overridden to {N})" if args.rows else "")
                        + f": {w.head} fwd+bwd, "
                        f"{'bf16' if es == 2 else 'fp32'} logits [{N}, {V}]"
                        + (f", k={w.k}" if w.head == "logp" else "")
                        + ((", forward KL(ref||policy)" if args.direction else
                            ", reverse KL(policy||ref)") if w.head == "kl" else "")
                        + (f", softcap {w.cap:g}" if w.cap else ""),
            "N": N, "V": V, "logits_dtype": "bf16" if es == 2 else "fp32",
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_step": step_bytes,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        **({"softcap_standalone": time_softcap(args.workload, dev, torch)}
           if "softcap_shape" in w.extra else {}),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
