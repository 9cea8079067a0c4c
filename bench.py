#!/usr/bin/env python3
"""Benchmark: the fused log-softmax heads forward + backward on one MI355X.

A step is one forward + backward pass of the hot path over one batch of a
workload: the single-read row statistics with the head outputs (rlk_*_fwd),
then the fused zero-workspace backward (rlk_*_bwd), on seeded synthetic inputs
already resident in HBM.  By default every workload is timed in this one
process:

  c1_logp_fp32      logprobs k=1, fp32 [64, 32000]
  c2_logp_bf16      logprobs k=1, bf16 [8192, 151936]
  c3_kl_bf16        reverse KL and forward KL (timed apart), bf16 [8192, 75968] x 2
  c4_entropy_cap30  entropy with softcap 30, bf16 [32768, 151936]   (headline)
  c5_topk_cap20     top-256 logprobs with softcap 20, bf16 [2048, 262144],
                    plus the standalone softcap on bf16 [2, 3, 262144]

Prints ONE JSON line.  Its top-level figures are the headline workload's (the
largest one that fits one GPU): throughput in algorithmic GB/s (each logit
read once by the forward, read once and written once by the backward, plus
the per-row side arrays), the dominant kernel's roofline figures measured with
HIP events on the launch stream, and the fp64 CPU oracle timed on a bounded
sample of the same workload on the host cores.  ``configs`` holds the same
figures for every workload; ``provenance`` the build, device and software.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
METRIC = "fwd+bwd ms and HBM GB/s (% of 8 TB/s) for logp/entropy/KL at N x V"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "vocab_log_softmax_amd", "csrc")
BUILD_INFO = os.path.join(ROOT, "vocab_log_softmax_amd", "build_info.json")
HEADLINE = "c4_entropy_cap30"
# (workload, KL direction) in the order they are timed
ALL_RUNS = [("c1_logp_fp32", 0), ("c2_logp_bf16", 0), ("c3_kl_bf16", 0), ("c3_kl_bf16", 1),
            ("c4_entropy_cap30", 0), ("c5_topk_cap20", 0)]
# The oracle sample of each workload: at most this many logits per tensor
# (fp64 copies on the host), repeated until it has run for ORACLE_SECONDS.
ORACLE_MAX_ELEMS = 1 << 28
ORACLE_SECONDS = 2.0
ORACLE_MAX_THREADS = 16


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, kernel: str, which: str = "bwd"):
    """HBM bytes per launch of the workload's backward (or forward, which =
    "fwd") from the committed rocprofv3 --pmc summary named after its
    backward kernel, or None.

    The summary must name the same kernel sources (hash) as this tree; a
    changed kernel makes its counters stale.
    """
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    pre = "fwd_" if which == "fwd" else ""
    m_hash = re.search(r"^source_hash:\s*(\S+)", txt, re.M)
    m_rd = re.search(rf"^{pre}hbm_read_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    m_wr = re.search(rf"^{pre}hbm_write_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
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
        self.hip = hip_runtime(torch)
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


def hip_runtime(torch):
    """The HIP runtime library torch loaded (same soname -> same instance)."""
    lib_dir = os.path.join(os.path.dirname(torch.__file__), "lib")
    path = os.path.join(lib_dir, "libamdhip64.so")
    return ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")


def provenance(torch, dev) -> dict:
    """Where a record comes from: build, sources, device, software, host."""
    info: dict = {"source_hash": kernel_source_hash()}
    try:
        with open(BUILD_INFO) as f:
            bi = json.load(f)
        info["git_commit"] = bi.get("git_commit")
        info["git_dirty"] = bi.get("git_dirty")
        info["library_built_from_sources"] = bi.get("source_hash")
        info["library_matches_sources"] = bi.get("source_hash") == info["source_hash"]
    except (OSError, ValueError):
        info["git_commit"] = None
        info["library_matches_sources"] = None
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    info["torch"] = torch.__version__
    info["torch_hip"] = getattr(torch.version, "hip", None)
    hip = hip_runtime(torch)
    v = ctypes.c_int()
    if hip.hipRuntimeGetVersion(ctypes.byref(v)) == 0:
        info["hip_runtime_version"] = v.value
    if hip.hipDriverGetVersion(ctypes.byref(v)) == 0:
        info["hip_driver_version"] = v.value
    p = torch.cuda.get_device_properties(dev)
    info["device"] = p.name
    info["arch"] = getattr(p, "gcnArchName", None)
    info["compute_units"] = p.multi_processor_count
    info["device_memory_gib"] = round(p.total_memory / 2**30, 1)
    info["host"] = {"cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
                    "machine": platform.machine(), "python": platform.python_version()}
    return info


def measure_ceilings(w, dev, torch) -> dict:
    """Practical HBM ceilings at the workload's tensor size (libceiling.so).

    Read-only, write-only and copy streams of 16-byte nontemporal accesses,
    grid-stride and row by row (one workgroup per row of V logits, as the
    library's kernels stream), and reads by one-shot workgroups that each
    fold one 16, 32 or 64 KB piece of a row; median of 15 timed launches
    after 3 warm-up launches, HIP events on the current stream.
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
             "read_rows": (3, 1), "copy_rows": (4, 2), "read_pieces_16k": (5, 1),
             "read_pieces_32k": (6, 1), "read_pieces_64k": (7, 1)}
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


def measure_launch_floor(dev, torch) -> dict:
    """Latency probes at the logprobs fp32 [64, 32000] size (libceiling.so):
    back-to-back launch intervals of empty kernels, a one-workgroup-per-row
    read with every load in flight, the same with the row kernels' online
    fold and with their epilogue, the fold split over four workgroups per
    row (alone, and with a last-arriver combine and the epilogue in the same
    launch), the backward's one-shot pieces, and pairs of them; beside them the
    library's own forward, backward and step on the workload; and the empty
    pair and the library's step replayed from HIP graphs of 10 steps.  Each
    figure is the best of 5 runs of 500 back-to-back launches or steps (HIP
    events, mean per launch or step); the probes are launched from a C loop,
    the library through its binding (about 3 us of host time per call, under
    the GPU time here)."""
    from vocab_log_softmax_amd import build as B
    from vocab_log_softmax_amd import rlk, workloads

    if not os.path.exists(B.CEILING_LIB):
        raise SystemExit(f"{B.CEILING_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(B.CEILING_LIB)
    lib.launch_floor_run.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 6
    lib.launch_floor_run.restype = ctypes.c_int
    R, C = lib.launch_floor_rows(), lib.launch_floor_cols()
    d = workloads.make_inputs("c1_logp_fp32", dev)
    x = d["logits"]
    assert tuple(x.shape) == (R, C) and x.dtype == torch.float32
    y = torch.empty_like(x)
    tg = d["targets"].reshape(-1).contiguous()
    stats = torch.empty(R * 8, dtype=torch.float32, device=dev)
    out = torch.empty(256, dtype=torch.float32, device=dev)
    raw = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ev = HipEvents(2, torch)

    def probe(a, b=-1):
        def run(reps):
            rc = lib.launch_floor_run(a, b, reps, x.data_ptr(), y.data_ptr(), tg.data_ptr(),
                                      stats.data_ptr(), out.data_ptr(), raw)
            if rc != 0:
                raise RuntimeError(f"launch_floor_run({a}, {b}) failed: {rc}")
        return run

    def best_us(run, reps=500, per=1):
        run(max(1, reps // 10))
        best = float("inf")
        for _ in range(5):
            torch.cuda.synchronize()
            ev.record(0, raw)
            run(reps)
            ev.record(1, raw)
            torch.cuda.synchronize()
            best = min(best, ev.elapsed_ms(0, 1) * 1e3 / reps / per)
        return round(best, 2)

    names = ["empty, 64 workgroups", "empty, 1024 workgroups",
             "row read, one workgroup per row, every load in flight",
             "row read + online fold", "row read + fold + forward epilogue",
             "fold split over 4 workgroups per row", "backward-shaped one-shot pieces (copy)",
             "fold split over 4 workgroups per row + last-arriver combine and epilogue"]
    res = {n: best_us(probe(k)) for k, n in enumerate(names)}
    res["pair: empty + empty"] = best_us(probe(0, 1))
    res["pair: read + fold + epilogue, then one-shot pieces"] = best_us(probe(4, 6))
    res["pair: split + combine, then one-shot pieces"] = best_us(probe(7, 6))
    tg2, g = d["targets"], d["grad"]
    lp = torch.empty(tg2.shape, dtype=torch.float32, device=dev)
    st = rlk.new_stats(rlk.RLK_HEAD_LOGP, R, C, dev)
    gx = torch.empty_like(x)
    fwd = rlk.prepare(rlk.rlk_logp_fwd, x, tg2, 0.0, lp, st)
    bwd = rlk.prepare(rlk.rlk_logp_bwd, x, tg2, 0.0, st, g, gx)
    def loop(*fns):  # the library through its Python binding (host-side ~3 us per call)
        def run(reps):
            for _ in range(reps):
                for f in fns:
                    f()
        return run

    res["library: logprobs forward"] = best_us(loop(fwd))
    res["library: logprobs backward"] = best_us(loop(bwd))
    res["library: forward + backward step"] = best_us(loop(fwd, bwd))

    # The same pairs from HIP graphs of G steps (one graph launch per G
    # steps): dependent kernels without a stream launch each.  Every replay
    # of the library's graph is compared bit for bit with the eager step,
    # with eager work between the replays.
    G = 10

    def graph(capture):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            capture()
        return gr

    def empty_pairs():
        cs = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        rc = lib.launch_floor_run(0, 0, G, x.data_ptr(), y.data_ptr(), tg.data_ptr(),
                                  stats.data_ptr(), out.data_ptr(), cs)
        if rc != 0:
            raise RuntimeError(f"launch_floor_run under capture failed: {rc}")

    def library_steps():
        f = rlk.prepare(rlk.rlk_logp_fwd, x, tg2, 0.0, lp, st)
        b = rlk.prepare(rlk.rlk_logp_bwd, x, tg2, 0.0, st, g, gx)
        for _ in range(G):
            f()
            b()

    g_empty, g_lib = graph(empty_pairs), graph(library_steps)
    fwd()
    bwd()
    torch.cuda.synchronize()
    ref_lp, ref_gx = lp.clone(), gx.view(torch.int32).clone()
    for _ in range(3):
        lp.zero_()
        gx.zero_()
        g_lib.replay()
        torch.cuda.synchronize()
        if not (torch.equal(lp, ref_lp) and torch.equal(gx.view(torch.int32), ref_gx)):
            raise RuntimeError("a graph replay differs from the eager step")
        fwd()
        bwd()
        torch.cuda.synchronize()

    def replays(gr):
        def run(reps):
            for _ in range(reps):
                gr.replay()
        return run

    res[f"graph of {G} pairs: empty + empty, per pair"] = best_us(replays(g_empty), 50, G)
    res[f"graph of {G} library steps: per step"] = best_us(replays(g_lib), 50, G)
    ev.close()
    return {"launch_floor_us": res, "shape": [R, C], "dtype": "fp32",
            "method": "best of 5 x 500 back-to-back launches (or graph-replayed steps), HIP "
                      "events, mean per launch or step; probes launched from a C loop"}


def measure_issue_rate(dev, torch) -> dict:
    """VALU issue rates (libceiling.so): wave64 FMA, v_exp_f32 and v_rcp_f32
    with 8 independent chains per lane at 4, 8 and 16 waves per SIMD
    (256-thread workgroups).  Reported as cycles per wave instruction per
    SIMD at the 2.4 GHz peak engine clock, best of 6 launches each."""
    from vocab_log_softmax_amd import build as B

    if not os.path.exists(B.CEILING_LIB):
        raise SystemExit(f"{B.CEILING_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(B.CEILING_LIB)
    lib.issue_rate_run.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2
    lib.issue_rate_run.restype = ctypes.c_int
    iters = 4096
    simds = torch.cuda.get_device_properties(dev).multi_processor_count * 4
    out = torch.empty(4 * simds * 256, dtype=torch.float32, device=dev)
    raw = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ev = HipEvents(2, torch)
    res = {}
    for waves in (4, 8, 16):  # waves per SIMD: 256-thread workgroups of 4 waves
        blocks = waves * simds // 4
        wave_instr = blocks * 4 * iters * lib.issue_rate_chains()  # per launch
        r = {}
        for op, name in enumerate(("fma", "exp2", "rcp")):
            best = float("inf")
            for _ in range(6):
                torch.cuda.synchronize()
                ev.record(0, raw)
                rc = lib.issue_rate_run(op, blocks, iters, ctypes.c_void_p(out.data_ptr()), raw)
                ev.record(1, raw)
                torch.cuda.synchronize()
                if rc != 0:
                    raise RuntimeError(f"issue_rate_run({op}) failed: {rc}")
                best = min(best, ev.elapsed_ms(0, 1))
            cycles = best * 1e-3 * 2.4e9 * simds / wave_instr
            r[name] = {"ms": round(best, 4), "cycles_per_wave_instr_per_simd": round(cycles, 2)}
        r["transcendental_vs_fma"] = round(r["exp2"]["cycles_per_wave_instr_per_simd"] /
                                           r["fma"]["cycles_per_wave_instr_per_simd"], 2)
        res[f"{waves}_waves_per_simd"] = r
    ev.close()
    return {"issue_rate": res, "iterations": iters, "chains_per_lane": lib.issue_rate_chains(),
            "simds": simds}


def time_softcap(name: str, dev, torch, reps: int = 200) -> dict:
    """The standalone softcap forward (y fp32) and backward on the workload's
    softcap tensor: mean kernel time over `reps` back-to-back launches, HIP
    events."""
    from vocab_log_softmax_amd import rlk, workloads

    w = workloads.WORKLOADS[name]
    x, gy = workloads.make_softcap_inputs(name, dev)
    y = torch.empty(x.shape, dtype=torch.float32, device=dev)
    gx = torch.empty_like(x)
    n, es = x.numel(), x.element_size()
    raw = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    out = {"shape": list(x.shape), "dtype": str(x.dtype).replace("torch.", ""), "cap": w.cap,
           "reps": reps}
    fwd = rlk.prepare(rlk.rlk_softcap_fwd, x, y, w.cap)
    bwd = rlk.prepare(rlk.rlk_softcap_bwd, x, gy, gx, w.cap)
    for what, fn, nbytes in (("fwd", fwd, n * (es + 4)), ("bwd", bwd, n * (es + 4 + es))):
        for _ in range(20):
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
    tot = out["fwd"]["us"] + out["bwd"]["us"]
    out["fwd+bwd_us"] = round(tot, 2)
    out["GB/s"] = round((out["fwd"]["bytes"] + out["bwd"]["bytes"]) / (tot * 1e-6) / 1e9, 1)
    out["frac_of_hbm_peak"] = round(out["GB/s"] / HBM_PEAK_GBS, 4)
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


def oracle_baseline(w, d, direction: int, step_bytes: int, threads: int) -> dict:
    """The fp64 oracle's fwd+bwd on the first rows of the same inputs.

    At most ORACLE_MAX_ELEMS logits per tensor; the pass is repeated until
    ORACLE_SECONDS have elapsed (at most 1000 passes) and the mean time of
    one pass is reported, scaled to GB/s of the workload's algorithmic bytes.
    """
    import oracle

    orc = oracle.get()
    orc.set_threads(threads)
    N, V = d["N"], d["V"]
    n = max(1, min(N, ORACLE_MAX_ELEMS // V))
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
        if dt >= ORACLE_SECONDS or passes >= 1000:
            break
    per_pass = dt / passes
    return {"value": round(step_bytes * n / N / per_pass / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "host_affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"fp64 oracle fwd+bwd (OpenMP, {threads} threads) on the first {n} of {N} "
                      f"rows of the same workload ({n * V} logits per tensor): "
                      f"{per_pass:.4f} s per pass, mean of {passes} "
                      f"pass{'es' if passes > 1 else ''} ({dt:.1f} s)"}


def setup_workload(name, direction, dev, torch, rows=None):
    """Inputs, outputs and pre-marshalled fwd / bwd calls of one workload."""
    from vocab_log_softmax_amd import rlk, workloads

    w = workloads.WORKLOADS[name]
    d = workloads.make_inputs(name, dev, N=rows)
    x = d["logits"]
    N, V = x.shape
    es = x.element_size()
    gx = torch.empty_like(x)
    if w.head == "logp":
        tg, g = d["targets"], d["grad"]
        out = torch.empty(tg.shape, dtype=torch.float32, device=dev)
        st = rlk.new_stats(rlk.RLK_HEAD_LOGP, N, V, dev)
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
        fwd = rlk.prepare(rlk.rlk_entropy_fwd, x, w.cap, out, st)
        bwd = rlk.prepare(rlk.rlk_entropy_bwd, x, w.cap, st, g, gx)
        n_in, fwd_name, bwd_name = 1, fwd1_name(w, N, V, es), "bwd_piece_kernel"
    else:
        ref, g = d["ref"], d["grad"]
        out = torch.empty(N, dtype=torch.float32, device=dev)
        st = rlk.new_stats(rlk.RLK_HEAD_KL, N, V, dev)
        fwd = rlk.prepare(rlk.rlk_kl_fwd, x, ref, direction, 0.0, 0.0, out, st)
        bwd = rlk.prepare(rlk.rlk_kl_bwd, x, ref, direction, 0.0, 0.0, st, g, gx)
        n_in, fwd_name, bwd_name = 2, "fwdkl_kernel", "bwd_piece_kernel"
    sf, sb = side_bytes(w, N)
    fwd_bytes = n_in * N * V * es + sf            # read every input logit once
    bwd_bytes = (n_in + 1) * N * V * es + sb      # read again, write the gradient once
    desc = (f"{name}: {w.head} fwd+bwd, {'bf16' if es == 2 else 'fp32'} logits [{N}, {V}]"
            + (f" x 2" if w.head == "kl" else "")
            + (f", k={w.k}" if w.head == "logp" else "")
            + ((", forward KL(ref||policy)" if direction else ", reverse KL(policy||ref)")
               if w.head == "kl" else "")
            + (f", softcap {w.cap:g}" if w.cap else ""))
    keep = (x, gx, out, st, d)
    return dict(w=w, d=d, N=N, V=V, es=es, fwd=fwd, bwd=bwd, fwd_name=fwd_name,
                bwd_name=bwd_name, fwd_bytes=fwd_bytes, bwd_bytes=bwd_bytes, desc=desc,
                keep=keep)


def time_steps(fwd, bwd, stream, torch, steps=None, warmup=None, cold=False, dev=None) -> dict:
    """Warm up, then time `steps` back-to-back fwd+bwd steps (wall clock) with
    HIP events around the forward and the backward of sampled steps.

    Without explicit counts both are sized from the step time: a
    launch-bound step (microseconds) needs thousands of steps before clocks
    and queues settle and for the timed region to outweigh its start-up
    (warm-up >= 50 ms, timed region >= 0.2 s, at least 50 steps).
    """
    def run(n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fwd()
            bwd()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / max(1, n)

    if warmup is not None:
        warm_ms = run(warmup)
    else:
        run(5)                   # first launches (code loading, clocks)
        warm_ms = run(10)        # the step time, from settled launches
        extra = max(0, math.ceil(50.0 / max(warm_ms, 1e-6)) - 15)
        run(extra)
        warmup = 15 + extra
    if steps is None:
        steps = max(50, math.ceil(200.0 / max(warm_ms, 1e-6)))

    # Three events per sampled step: before the forward, between forward and
    # backward, after the backward.  Every step is sampled unless a step is
    # so short (launch-bound) that the markers would show in its wall time;
    # then every tenth step is.
    stride = 1 if (warm_ms > 0.2 or cold) else 10
    sampled = list(range(0, steps, stride))
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev) if cold else None
    ev = HipEvents(3 * len(sampled), torch)
    raw = ctypes.c_void_p(stream.cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    j = 0
    for i in range(steps):
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
    del flush
    ms_per_step = wall * 1e3 / steps
    if cold:  # the flush is not part of a step: the kernels' event time
        ms_per_step = fwd_ms + bwd_ms
    return dict(steps=steps, warmup=warmup, ms_per_step=ms_per_step, fwd_ms=fwd_ms,
                bwd_ms=bwd_ms, event_timed_steps=len(sampled))


def run_workload(name, direction, dev, torch, args, steps=None, warmup=None) -> dict:
    """Time one workload; returns its record (and the roofline of its
    dominant kernel)."""
    s = setup_workload(name, direction, dev, torch, rows=args.rows)
    stream = torch.cuda.current_stream(dev)
    tm = time_steps(s["fwd"], s["bwd"], stream, torch, steps=steps, warmup=warmup,
                    cold=args.cold, dev=dev)
    step_bytes = s["fwd_bytes"] + s["bwd_bytes"]
    value = step_bytes / (tm["ms_per_step"] * 1e-3) / 1e9
    fwd_gbs = s["fwd_bytes"] / (tm["fwd_ms"] * 1e-3) / 1e9
    bwd_gbs = s["bwd_bytes"] / (tm["bwd_ms"] * 1e-3) / 1e9
    # traffic summaries are per workload (and per direction for KL)
    pkey = None
    if args.rows is None:
        pkey = name + ({0: "_reverse", 1: "_forward"}[direction] if s["w"].head == "kl" else "")
    t_bwd = traffic_from_profiles(pkey, s["bwd_name"]) if pkey else None
    t_fwd = traffic_from_profiles(pkey, s["bwd_name"], "fwd") if pkey else None
    # the dominant kernel: the one with the longer event time
    dom_bwd = tm["bwd_ms"] >= tm["fwd_ms"]
    k_name, k_ms, k_bytes, k_gbs = ((s["bwd_name"], tm["bwd_ms"], s["bwd_bytes"], bwd_gbs)
                                    if dom_bwd else
                                    (s["fwd_name"], tm["fwd_ms"], s["fwd_bytes"], fwd_gbs))
    other = ((s["fwd_name"], "forward", tm["fwd_ms"], s["fwd_bytes"], fwd_gbs) if dom_bwd else
             (s["bwd_name"], "backward", tm["bwd_ms"], s["bwd_bytes"], bwd_gbs))
    head = s["w"].head
    roofline = {
        "bound": "hbm",
        "kernel": f"{k_name} ({head} {'backward' if dom_bwd else 'forward'})",
        "achieved": round(k_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(k_gbs / HBM_PEAK_GBS, 4),
        "traffic": t_bwd if dom_bwd else t_fwd,
        "algorithmic_bytes_per_launch": k_bytes,
        "avg_launch_ms": round(k_ms, 4),
        "event_timed_steps": tm["event_timed_steps"],
        "second_kernel": {"kernel": f"{other[0]} ({head} {other[1]})",
                          "avg_launch_ms": round(other[2], 4), "achieved": round(other[4], 1),
                          "frac": round(other[4] / HBM_PEAK_GBS, 4),
                          "algorithmic_bytes_per_launch": other[3]},
    }
    rec = {
        "workload": s["desc"], "N": s["N"], "V": s["V"],
        "logits_dtype": "bf16" if s["es"] == 2 else "fp32", "seed": s["w"].seed,
        "steps": tm["steps"], "warmup": tm["warmup"],
        "ms_per_step": round(tm["ms_per_step"], 5),
        "fwd_ms": round(tm["fwd_ms"], 5), "bwd_ms": round(tm["bwd_ms"], 5),
        "GB/s": round(value, 1), "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "fwd_GB/s": round(fwd_gbs, 1), "bwd_GB/s": round(bwd_gbs, 1),
        "algorithmic_bytes_per_step": step_bytes,
        "traffic_ratio_fwd": (round(t_fwd / s["fwd_bytes"], 4) if t_fwd else None),
        "traffic_ratio_bwd": (round(t_bwd / s["bwd_bytes"], 4) if t_bwd else None),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        threads = args.oracle_threads or min(len(os.sched_getaffinity(0)), ORACLE_MAX_THREADS)
        rec["cpu_baseline"] = oracle_baseline(s["w"], s["d"], direction, step_bytes, threads)
    if "softcap_shape" in s["w"].extra and args.rows is None:
        rec["softcap_standalone"] = time_softcap(name, dev, torch)
    del s
    torch.cuda.empty_cache()
    return rec


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps of the headline workload (default: at least 50, enough "
                         "for 0.2 s of work; the other workloads always size their own)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: at least 5, enough for 50 ms)")
    ap.add_argument("--workload", default=None,
                    help="time this workload only (default: every workload, headline "
                         f"{HEADLINE})")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-threads", type=int, default=None,
                    help="host threads of the CPU oracle (default: the process's cores, "
                         f"at most {ORACLE_MAX_THREADS})")
    ap.add_argument("--rows", type=int, default=None,
                    help="with --workload: override the row count N (same recipe, e.g. 32768 "
                         "rows of c2_logp_bf16 for the pages' B200 comparison)")
    ap.add_argument("--direction", type=int, default=0, choices=(0, 1),
                    help="with a KL --workload: 0 reverse KL(policy||ref), 1 forward "
                         "KL(ref||policy)")
    ap.add_argument("--cold", action="store_true",
                    help="write a 1 GiB buffer before every step (flushes the 256 MB Infinity "
                         "Cache and the L2s) and time the two kernels with events only")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the read / write / copy ceilings at the workload's size")
    ap.add_argument("--launch-floor", action="store_true",
                    help="only measure the launch-latency probes at the fp32 [64, 32000] size")
    ap.add_argument("--issue-rate", action="store_true",
                    help="only measure the VALU issue rates of FMA, exp2 and rcp")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of a known size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(rows shard across GPUs with no exchange; vocabulary shards need one "
              "all-gather of the rlk_*_fwd_partial records before rlk_combine). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.rows is not None and args.workload is None:
        print("--rows needs --workload", file=sys.stderr)
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
    if args.launch_floor:
        print(json.dumps(measure_launch_floor(dev, torch)))
        return 0
    if args.issue_rate:
        print(json.dumps(measure_issue_rate(dev, torch)))
        return 0
    if args.ceilings:
        w = workloads.WORKLOADS[args.workload or HEADLINE]
        print(json.dumps(measure_ceilings(w, dev, torch)))
        return 0

    if args.workload is not None:
        runs = [(args.workload, args.direction)]
        headline = runs[0]
    else:
        runs = ALL_RUNS
        headline = (HEADLINE, 0)
    configs = {}
    for name, direction in runs:
        is_head = (name, direction) == headline
        rec = run_workload(name, direction, dev, torch, args,
                           steps=args.steps if is_head else None,
                           warmup=args.warmup if is_head else None)
        key = name + ({0: "_reverse", 1: "_forward"}[direction]
                      if workloads.WORKLOADS[name].head == "kl" else "")
        configs[key] = rec
        print(f"[bench] {key}: {rec['ms_per_step']:.5f} ms/step, {rec['GB/s']} GB/s "
              f"({100 * rec['frac_of_hbm_peak']:.1f}% of 8 TB/s)", file=sys.stderr, flush=True)
    hkey = headline[0] + ({0: "_reverse", 1: "_forward"}[headline[1]]
                          if workloads.WORKLOADS[headline[0]].head == "kl" else "")
    h = configs[hkey]
    result = {
        "metric": METRIC,
        "value": h["GB/s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": h["warmup"],
        "ms_per_step": round(h["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "timing": ("cold: 1 GiB written before every step, step = forward + backward event time"
                   if args.cold else "warm: back-to-back steps, wall clock"),
        "config": {
            "workload": h["workload"] + (f" (N overridden to {h['N']})" if args.rows else ""),
            "N": h["N"], "V": h["V"], "logits_dtype": h["logits_dtype"],
            "frac_of_hbm_peak": h["frac_of_hbm_peak"],
            "algorithmic_bytes_per_step": h["algorithmic_bytes_per_step"],
            "fwd_ms": h["fwd_ms"], "bwd_ms": h["bwd_ms"],
        },
        "roofline": h["roofline"],
        "cpu_baseline": h.get("cpu_baseline"),
        "configs": {k: {kk: vv for kk, vv in v.items() if kk != "roofline"}
                    | {"dominant_kernel": v["roofline"]["kernel"],
                       "dominant_kernel_frac": v["roofline"]["frac"]}
                    for k, v in configs.items()},
        "provenance": provenance(torch, dev),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
