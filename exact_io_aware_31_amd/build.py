"""Build libfa.so (the gfx950 attention library) in-tree with hipcc.

    python -m exact_io_aware_31_amd.build      # or build_library() from Python

Every source is compiled for gfx950 only.  All HIP code is compiled with
packed-fp32 instruction selection disabled (``-packed-fp32-ops``) and with
``-fno-honor-nans``: the library's contract requires finite inputs, which
lets max reductions compile to bare v_max/v_max3 without NaN-quieting
canonicalisations.
Output: exact_io_aware_31_amd/_lib/libfa.so (the attention library) and
exact_io_aware_31_amd/_lib/libfa_probe.so (the two measurement kernels of
include/fa_probe.h, used by the benchmark to measure the chip's own ceilings).

Every HIP source is compiled with the backend's kernel resource report; the
per-kernel registers, occupancy and scratch are written to
_build/kernel_resources.txt, and the build fails if any kernel spills to
scratch memory (a spill turns register traffic into memory traffic on every
loop iteration).
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libfa.so")
PROBE_LIB = os.path.join(LIB_DIR, "libfa_probe.so")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip"]
PROBE_SOURCES = ["fa_probe_api.cpp", "fa_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fno-honor-nans"]


def _resources(text: str):
    """(kernel, VGPRs, AGPRs, scratch bytes per lane, waves per SIMD) from the backend's
    kernel-resource-usage remarks."""
    out, cur = [], None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            out.append(cur)
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split()[0]] = int(m.group(2))
    return out


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [hipcc()] + common_flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is expected.
    noise = "is not a recognized feature for this target"
    text = r.stdout + r.stderr
    msgs = [ln for ln in text.splitlines()
            if noise not in ln and "kernel-resource-usage" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    if src.endswith(".hip"):
        with open(obj + ".resources", "w") as f:
            for k in _resources(text):
                f.write(f"{k['name']} vgpr={k.get('VGPRs', -1)} agpr={k.get('AGPRs', -1)} "
                        f"scratch={k.get('ScratchSize', -1)} waves_per_simd={k.get('Occupancy', -1)}\n")
    return obj


def _check_resources(objs) -> None:
    """Write _build/kernel_resources.txt; fail if a kernel uses scratch memory."""
    lines = []
    for o in objs:
        if os.path.exists(o + ".resources"):
            lines += open(o + ".resources").read().splitlines()
    with open(os.path.join(BUILD_DIR, "kernel_resources.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    spills = [ln for ln in lines if "scratch=0 " not in ln]
    if spills:
        raise RuntimeError("kernels using scratch memory (register spills):\n" + "\n".join(spills))


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    _check_kernel_stubs(tmp)
    os.replace(tmp, lib)


def build_library(verbose: bool = False) -> str:
    """Compile and link libfa.so and libfa_probe.so; returns the path of libfa.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + PROBE_SOURCES))
    _check_resources(objs)
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


def _check_kernel_stubs(lib: str) -> None:
    """Fail if a kernel's host-side launch stub is undefined.

    When the host pass cannot analyse a kernel body (for example a target
    builtin called directly in it rather than through a __device__ helper),
    hipcc drops the kernel's host stub without an error; the library then
    links but cannot be loaded.  Catch that at build time."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    r = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    if r.returncode != 0:
        return  # no nm available: skip the check rather than fail the build
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        raise RuntimeError(f"kernel launch stubs missing from {os.path.basename(lib)}: "
                           + ", ".join(missing))


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
