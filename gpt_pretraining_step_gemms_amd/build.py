"""Builds libncgpt.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m gpt_pretraining_step_gemms_amd.build   (or __graft_entry__.build())
"""

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libncgpt.so")
SOURCES = ["gemm.hip", "attention.hip", "elementwise.hip", "extras.hip", "runtime.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    # packed fp32 ops are kept off (plain fp32 VALU code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}",
]


def _torch_lib_dir():
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec and spec.origin:
            return os.path.join(os.path.dirname(spec.origin), "lib")
    except Exception:
        pass
    return None


def build(verbose=True, jobs=4):
    os.makedirs(OBJ, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        while sum(p.poll() is None for _, p in procs) >= jobs:
            time.sleep(0.2)
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(f"--- {src} ---\n{out}\n")
        elif verbose and out.strip():
            sys.stderr.write(out + "\n")
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    tl = _torch_lib_dir()
    if tl:
        # resolve libamdhip64 to the copy torch loads, so both share one HIP runtime
        link.append(f"-Wl,-rpath,{tl}")
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build()
