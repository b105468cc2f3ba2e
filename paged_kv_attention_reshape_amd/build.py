"""Build the HIP libraries in-tree for gfx950.

  libpa.so            paged_kv_attention_reshape_amd/  (the attention library)
  libpa_sched.so      paged_kv_attention_reshape_amd/  (host scheduler / block
                                                        allocator, plain C++)
  libpa_workloads.so  workloads/                        (device input generator,
                                                        test/benchmark only)

Every HIP translation unit is compiled with packed-fp32 instruction selection
turned off (the -packed-fp32-ops target feature) so that no v_pk_*_f32 is
emitted.  Usage: python -m paged_kv_attention_reshape_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
BUILD_DIR = os.path.join(ROOT, "_build")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-file extra flags.  The chunk kernel's scores never hold a NaN (masked
# rows re-read finite cache rows), so max/min need no NaN canonicalisation;
# infinities are still honoured (the causal mask uses -inf).
EXTRA_FLAGS = {"k_chunk.hip": ["-fno-honor-nans"]}


def _compile(src: str, obj: str, includes, verbose: bool) -> None:
    extra = EXTRA_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC, *COMMON, *extra, *[f"-I{i}" for i in includes], "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {out}:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)


def _build_lib(name: str, srcs, includes, out: str, verbose: bool) -> str:
    bdir = os.path.join(BUILD_DIR, name)
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], includes, verbose), zip(srcs, objs)))
    _link(objs, out, verbose)
    return out


CXX = os.environ.get("CXX", "g++")


def _build_host_lib(srcs, includes, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [CXX, "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", *[f"-I{i}" for i in includes],
           *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host build failed for {out}:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False):
    inc = [os.path.join(ROOT, "include"), os.path.join(PKG, "csrc")]
    sched = _build_host_lib([os.path.join(PKG, "csrc", "sched.cpp")], [os.path.join(ROOT, "include")],
                            os.path.join(PKG, "libpa_sched.so"), verbose)
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    lib = _build_lib("pa", srcs, inc, os.path.join(PKG, "libpa.so"), verbose)
    wsrcs = sorted(glob.glob(os.path.join(ROOT, "workloads", "csrc", "*.hip")))
    wlib = _build_lib("workloads", wsrcs, [], os.path.join(ROOT, "workloads", "libpa_workloads.so"), verbose)
    return lib, wlib, sched


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
