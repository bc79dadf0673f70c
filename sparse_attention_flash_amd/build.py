"""Build libsa_hip.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python sparse_attention_flash_amd/build.py

Every ``csrc/*.hip`` file is compiled for gfx950 only and linked into one shared library next to
this file, and ``probes/*.hip`` (the peak-rate microbenchmarks of include/sa_probes.h) into
libsa_probes.so beside it.  Packed-fp32 instruction selection is disabled for all device code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libsa_hip.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
PROBES_LIB_PATH = os.path.join(PKG, "libsa_probes.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # let MFMA accumulate in VGPRs so softmax arithmetic on S needs no AGPR round trips
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libsa_hip.so")
    return path


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (libsa_hip_san.so): the C ABI's
# argument checks, planning and launch code run instrumented; device code is built as usual.  The
# shared ASan runtime must be preloaded into the host process (tests/run_cpu_tests_sanitized.sh).
SAN_LIB_NAME = "libsa_hip_san.so"
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source and link libsa_hip.so (libsa_hip_san.so with sanitize=True), and
    libsa_probes.so unless sanitizing; returns the attention library's path."""
    lib_path = os.path.join(PKG, SAN_LIB_NAME) if sanitize else LIB_PATH
    _link(sources(), "_build_san" if sanitize else "_build", lib_path, sanitize, verbose)
    if not sanitize:
        _link(sorted(glob.glob(os.path.join(PKG, "probes", "*.hip"))), "_build_probes",
              PROBES_LIB_PATH, False, verbose)
    return lib_path


def _link(srcs, objdir_name, lib_path, sanitize, verbose):
    objdir = os.path.join(PKG, objdir_name)
    extra = SAN_HOST_FLAGS if sanitize else []
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag; that note is harmless
        text = "\n".join(ln for ln in text.splitlines() if "packed-fp32-ops" not in ln)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = lib_path + f".tmp{os.getpid()}"
    link_extra = [*extra, "-shared-libasan"] if sanitize else []
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs,
                    "-o", tmp], check=True)
    os.replace(tmp, lib_path)


if __name__ == "__main__":
    t0 = time.time()
    path = build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
    print(f"built {path} in {time.time() - t0:.1f}s")
