"""Build libpkv in-tree.

* ``lib/libpkv.so``      -- the full C-ABI library: host allocator + HIP
  kernels for gfx950 (hipcc), loaded by the Python binding.
* ``lib/libpkv_host.so`` -- the host allocator alone, compiled by g++ with no
  GPU code, for allocator tests on machines without a GPU.

Every HIP source is compiled with packed-FP32 instruction selection turned
off (the compiler would otherwise fuse float pairs into v_pk_* forms).
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
BUILD = os.path.join(ROOT, "_build")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"

HOST_SOURCES = ["host/pool.cpp", "host/plan.cpp", "host/plan_shared.cpp", "host/prepare.cpp", "host/prefill_plan.cpp",
                "host/utilisation.cpp", "host/hybrid.cpp", "host/sched.cpp"]
HIP_SOURCES = ["kernels/kv_write.hip", "kernels/paged_decode.hip", "kernels/paged_prefill.hip",
               "kernels/gather_probe.hip", "kernels/stepper.cpp"]

HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{INCLUDE}", "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", f"-I{INCLUDE}", "-Wall", "-Wextra"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device-only feature: harmless, filtered
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _obj(src, tag):
    return os.path.join(BUILD, tag, src.replace("/", "_") + ".o")


def build(verbose: bool = False) -> dict:
    """Compile both libraries; returns their paths."""
    os.makedirs(LIBDIR, exist_ok=True)
    for tag in ("dev", "host"):
        os.makedirs(os.path.join(BUILD, tag), exist_ok=True)
    jobs = []
    for s in HOST_SOURCES:
        jobs.append([CXX, *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", _obj(s, "host")])
    for s in HIP_SOURCES:
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", _obj(s, "dev")])
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    host_objs = [_obj(s, "host") for s in HOST_SOURCES]
    dev_objs = [_obj(s, "dev") for s in HIP_SOURCES]
    libpkv = os.path.join(LIBDIR, "libpkv.so")
    libhost = os.path.join(LIBDIR, "libpkv_host.so")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", libpkv + ".tmp",
          *dev_objs, *host_objs])
    os.replace(libpkv + ".tmp", libpkv)
    _run([CXX, "-shared", "-fPIC", "-o", libhost + ".tmp", *host_objs])
    os.replace(libhost + ".tmp", libhost)
    return {"libpkv": libpkv, "libpkv_host": libhost}


if __name__ == "__main__":
    print(build(verbose=True))
