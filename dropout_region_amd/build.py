"""Builds dropout_region_amd/libsp_region.so: the HIP kernels and the C ABI
of include/sp_region.h, compiled for gfx950 (MI355X) with hipcc.

Packed-fp32 instructions are switched off for all device code
(-target-feature -packed-fp32-ops); hipcc's host pass warns that it does not
know the feature, which is harmless.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsp_region.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["sp_fwd.hip", "sp_bwd.hip", "sp_region_api.hip", "ring_attn.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def build(out=LIB, verbose=False, extra=(), build_dir=BUILD_DIR):
    """Compiles every source in parallel, links the shared library, returns its
    path.  `extra` flags go on every compile and on the link (e.g. host-only
    sanitizers: -Xarch_host -fsanitize=...)."""
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        text = p.communicate()[0].decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{t}" for s, t in failed))
    tmp = out + ".tmp"
    subprocess.run([cc, "-shared", f"--offload-arch={ARCH}", *extra, "-o", tmp, *objs], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
