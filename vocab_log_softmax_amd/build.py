"""Compile the HIP library ``librlk.so`` for gfx950 (in-tree, next to this file).

Every translation unit under ``csrc/`` is compiled by hipcc in parallel and
linked into one shared library that exports the C ABI of ``include/rlk.h``.
Packed-fp32 instructions are disabled for all device code (the feature flag
below); hipcc's host pass prints that it does not know the feature, which is
harmless.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "librlk.so")
BUILD_INFO = os.path.join(PKG, "build_info.json")
# Bandwidth and launch-latency probes for the benchmark's ceiling reports
# (not part of the ABI).
CEILING_SRCS = [os.path.join(PKG, "ceiling", "ceiling.hip"),
                os.path.join(PKG, "ceiling", "launch_floor.hip"),
                os.path.join(PKG, "ceiling", "issue_rate.hip")]
CEILING_LIB = os.path.join(PKG, "ceiling", "libceiling.so")

SOURCES = ["rlk_fwd_f32.hip", "rlk_fwd_bf16.hip", "rlk_fwd_f16.hip",
           "rlk_bwd_f32.hip", "rlk_bwd_bf16.hip", "rlk_bwd_f16.hip",
           "rlk_softcap.hip", "rlk_combine.hip", "rlk_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, build_dir: str = BUILD_DIR, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines]]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", src if os.path.isabs(src) else os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def source_hash() -> str:
    """Hash of the kernel and host sources (the same rule as bench.py's)."""
    import hashlib

    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def write_build_info() -> None:
    """Record which commit and sources the library was built from.

    The GPU runs see the tree without its git metadata; the benchmark reports
    this file's commit, dirty flag and source hash as its provenance.
    """
    import json

    def git(*a):
        r = subprocess.run(["git", "-C", ROOT, *a], capture_output=True, text=True)
        return r.stdout.strip() if r.returncode == 0 else None

    status = git("status", "--porcelain", "--untracked-files=no")
    info = {"git_commit": git("rev-parse", "HEAD"),
            "git_dirty": None if status is None else bool(status),
            "source_hash": source_hash(), "arch": ARCH}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


def build(verbose: bool = True, out_path: str = LIB_PATH, defines=(), build_dir=BUILD_DIR) -> str:
    """Compile every source and link librlk.so; returns its path.

    ``defines`` (e.g. ``RLK_BLOCK=512``) override the launch-shape constants
    for tuning builds written to another ``out_path``.
    """
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), SOURCES))
    tmp = out_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out_path)
    if out_path == LIB_PATH and not defines:
        write_build_info()
    if verbose:
        print(f"built {out_path}")
    return out_path


def build_ceiling(verbose: bool = True) -> str:
    """Compile the bandwidth and launch-latency probes into libceiling.so
    (benchmark only)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [_compile(src, BUILD_DIR) for src in CEILING_SRCS]
    tmp = CEILING_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, CEILING_LIB)
    if verbose:
        print(f"built {CEILING_LIB}")
    return CEILING_LIB


if __name__ == "__main__":
    build()
    build_ceiling()
