"""Build libwallattn.so (gfx950) in-tree with hipcc.

    python -m exact_attention_channel_amd.build

The shared library lands next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "prefix.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_mfma.hip", "decode.hip", "decode_cache_bf16.hip",
           "decode_cache_f16.hip", "decode_cache_f32.hip"]
LIB = os.path.join(HERE, "libwallattn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # keep packed fp32 ops out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object in parallel (one hipcc per file),
    then link the shared library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    tag = "%d" % os.getpid()
    objs, procs = [], []
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".%s.o" % tag))
        objs.append(obj)
        procs.append(_run([hipcc(), *flags, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose))
    failed = False
    noise = "'-packed-fp32-ops' is not a recognized feature"
    for src, pr in zip(SOURCES, procs):
        out, _ = pr.communicate()
        msgs = [l for l in out.splitlines() if noise not in l]
        if pr.returncode != 0:
            failed = True
            sys.stderr.write(f"--- {src}\n" + "\n".join(msgs) + "\n")
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
        raise RuntimeError("hipcc failed building libwallattn.so")
    tmp = LIB + ".tmp" + tag
    res = subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                         capture_output=True, text=True)
    for o in objs:
        os.remove(o)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libwallattn.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
