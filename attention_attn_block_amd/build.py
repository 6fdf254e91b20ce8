"""Build libdit_attn.so in-tree for gfx950 with hipcc.

Each ``csrc/*.hip`` file compiles to an object in ``_build/`` (in parallel),
then one shared library is linked next to this file.  The measured-peak
micro-benchmarks in ``csrc/peaks/`` become a second library,
``libdit_peaks.so``, used only by the benchmark.  The plain-C client of
the ABI in ``tests/abi_client.c`` is then compiled with the host C compiler
and linked against that library.  Always recompiles.

    python -m attention_attn_block_amd.build
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdit_attn.so")
PEAKS_SRC = os.path.join(CSRC, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(HERE, "libdit_peaks.so")
ARCH = "gfx950"
CLIENT_SRC = os.path.join(ROOT, "tests", "abi_client.c")
CLIENT = os.path.join(ROOT, "tests", "abi_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

# Packed-fp32 VALU forms are disabled for all device code.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdit_attn.so)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False, jobs=None):
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in srcs]
    cmds = [[cc, *FLAGS, "-I", CSRC, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    # The measured-peak micro-benchmarks: a library of their own, for the benchmark.
    cmds.append([cc, *FLAGS, "-shared", PEAKS_SRC, "-o", PEAKS_LIB + ".tmp"])
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    os.replace(PEAKS_LIB + ".tmp", PEAKS_LIB)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    if os.path.exists(CLIENT_SRC):
        build_client(verbose)
    return LIB


def build_client(verbose=False):
    """Compile the C client of the ABI (C11, no HIP device code): it includes
    only include/dit_attn.h and links libdit_attn.so plus the HIP runtime."""
    cc = os.environ.get("CC") or shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no host C compiler found for tests/abi_client.c")
    tmp = CLIENT + ".tmp"
    _run([cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), CLIENT_SRC, "-o", tmp,
          "-L", HERE, "-ldit_attn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/../attention_attn_block_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    os.replace(tmp, CLIENT)
    if verbose:
        print("built", CLIENT)
    return CLIENT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
