"""Builds libpa.so in-tree with hipcc for gfx950 (MI355X).

    python -m paged_kv_cache_427_amd.build        # or: python paged_kv_cache_427_amd/build.py

Every HIP source is compiled with packed-fp32 instructions disabled (the compiler then emits only
scalar fp32 VALU math); objects go to paged_kv_cache_427_amd/_build/, the library to
paged_kv_cache_427_amd/libpa.so.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def sources():
    hip = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def _compile(src: str, device: bool):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + (DEVICE if device else ["-D__HIP_PLATFORM_AMD__"]) + ["-c", src, "-o", obj]
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, time.time() - t, r.stderr


def build(verbose: bool = True, jobs: int = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = sources()
    jobs = jobs or min(8, os.cpu_count() or 4)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, True) for s in hip] + [ex.submit(_compile, s, False) for s in cpp]
        for f in futs:
            obj, dt, err = f.result()
            objs.append(obj)
            if verbose:
                print(f"[build] {os.path.basename(obj)} {dt:.1f}s", flush=True)
                warn = [ln for ln in err.splitlines() if "warning" in ln and "packed-fp32-ops" not in ln]
                for ln in warn[:20]:
                    print("   ", ln)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
