"""Build librk_seg.so in-tree: host core with g++, gfx950 kernels with hipcc, linked by hipcc.

    python -m head_aware_paged_prefill_amd.build            # librk_seg.so
    python -m head_aware_paged_prefill_amd.build --checked  # librk_seg_checked.so

Every HIP line carries `-Xclang -target-feature -Xclang -packed-fp32-ops` (packed fp32 VALU ops off).

--checked builds the host core (allocator, tables, schedulers, the C ABI) with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer (-fno-sanitize-recover: the first finding aborts),
links it with the unchanged gfx950 kernel objects by g++, and writes librk_seg_checked.so beside the
normal build.  The kernels themselves are not instrumented.  Run the CPU suite against it with

    RK_SEG_LIB=head_aware_paged_prefill_amd/librk_seg_checked.so \
    LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
    python -m pytest tests -q -m "not gpu"

(the interpreter is not instrumented, so the ASan runtime is preloaded; leak reports would list the
interpreter's own allocations).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librk_seg.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
              "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd[:3]) + " ...")
    return r


HOST_SOURCES = ["rk_host.cpp", "rk_sched.cpp", "rk_sched_ops.cpp"]
HIP_SOURCES = ["rk_attn.hip", "rk_kernels.hip", "rk_mass.hip", "rk_decode.hip"]


def build(verbose: bool = False, out: str = LIB, extra_hip: list | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    objs = []
    for src in HOST_SOURCES:
        o = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        _run(["g++"] + HOST_FLAGS + inc + ["-c", os.path.join(CSRC, src), "-o", o], verbose)
        objs.append(o)
    objs += _hip_objects(inc, verbose, extra_hip)
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def _hip_objects(inc, verbose, extra_hip=None):
    objs = []
    for src in HIP_SOURCES:
        o = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        _run([HIPCC] + HIP_FLAGS + (extra_hip or []) + inc + ["-c", os.path.join(CSRC, src), "-o", o], verbose)
        objs.append(o)
    return objs


CHECKED_LIB = os.path.join(HERE, "librk_seg_checked.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build_checked(verbose: bool = False, out: str = CHECKED_LIB) -> str:
    """Host core under ASan + UBSan (g++), kernels as in build(), linked by g++ against the HIP runtime."""
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    objs = []
    for src in HOST_SOURCES:
        o = os.path.join(BUILD, os.path.splitext(src)[0] + ".checked.o")
        _run(["g++"] + HOST_FLAGS + SAN_FLAGS + inc + ["-c", os.path.join(CSRC, src), "-o", o], verbose)
        objs.append(o)
    objs += _hip_objects(inc, verbose)
    tmp = out + ".tmp"
    _run(["g++", "-shared", "-fPIC"] + SAN_FLAGS + objs + ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                                                        "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if "--checked" in sys.argv[1:]:
        print(build_checked(verbose=True))
    else:
        print(build(verbose=True))
