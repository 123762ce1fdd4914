"""Build libkvq.so (HIP kernels + C ABI) for gfx950 with hipcc.

    python -m paged_quantized_kv_kvq_amd.build [--jobs N] [--verbose]

Every .hip file under csrc/ is compiled to an object in csrc/../_build/, in
parallel, and linked into paged_quantized_kv_kvq_amd/libkvq.so; plain host
C++ (.cpp, the block manager) is compiled by the host compiler.  The cache
write is compiled with -ffp-contract=off: its codes must match a plain fp32
reference bit for bit, so no multiply-add may be fused.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
PROBE_SRC = os.path.join(HERE, "probe", "stream_read.hip")
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")   # measurement only: the streaming-read reference
INCLUDE = os.path.join(os.path.dirname(HERE), "include")  # the public C-ABI header
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the kvq library)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off (not needed; avoided on this target)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-command-line-argument",
]
EXACT = ["-ffp-contract=off"]          # bit-exact quantization
# decode: fused multiply-adds allowed; matrix-core accumulators kept in the
# ordinary VGPRs (the split pass rescales them between MFMAs, and AGPR
# accumulators would be copied out and back for every rescale)
FAST = ["-ffp-contract=fast", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def host_cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler found")


def compile_one(src: str, verbose: bool, out_dir: str = OUT_DIR, defines=()) -> tuple:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    if src.endswith(".cpp"):
        cmd = [host_cxx(), "-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", "-c", os.path.join(CSRC, src),
               "-o", obj]
    else:
        flags = EXACT if src in ("kvq_write.hip", "kvq_api.hip") else FAST
        cmd = [hipcc()] + COMMON + flags + [f"-I{INCLUDE}"] + [f"-D{d}" for d in defines] + \
            ["-c", os.path.join(CSRC, src), "-o", obj]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or r.returncode:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
    return src, obj, r.returncode, time.time() - t0


def _stale(src: str, out_dir: str) -> bool:
    """An object older than its source or than any header it may include."""
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(d, f) for d in (CSRC, INCLUDE) for f in os.listdir(d)
                                         if f.endswith(".h")]
    return max(os.path.getmtime(d) for d in deps) > os.path.getmtime(obj)


def build(jobs: int = 0, verbose: bool = False, lib: str = LIB, out_dir: str = OUT_DIR, defines=(),
          incremental: bool = False) -> str:
    """Compile and link.  `defines` (NAME=VALUE) override the tuning constants of
    csrc/kvq_internal.h; `lib` / `out_dir` place a variant build elsewhere;
    `incremental` recompiles only objects older than their inputs."""
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or max(1, min(8, os.cpu_count() or 1))
    objs = []
    failed = []
    todo = [s for s in sources() if not incremental or _stale(s, out_dir)]
    objs = [os.path.join(out_dir, os.path.splitext(s)[0] + ".o") for s in sources() if s not in todo]
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, obj, rc, dt in ex.map(lambda s: compile_one(s, verbose, out_dir, defines), todo):
            if verbose:
                sys.stderr.write(f"  {src}: {dt:.1f}s\n")
            (failed if rc else objs).append(src if rc else obj)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if lib == LIB and (not incremental or not os.path.exists(PROBE_LIB)
                       or os.path.getmtime(PROBE_SRC) > os.path.getmtime(PROBE_LIB)):
        build_probe(verbose)
    return lib


def build_probe(verbose: bool = False) -> str:
    """libkvq_probe.so: the streaming-read reference kernel the benchmark times."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc()] + COMMON + ["-O3", "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or r.returncode:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
    if r.returncode:
        raise RuntimeError("hipcc failed for the streaming-read probe")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--incremental", action="store_true", help="recompile only out-of-date objects")
    a = ap.parse_args()
    t0 = time.time()
    print(build(a.jobs, a.verbose, incremental=a.incremental), f"({time.time() - t0:.1f}s)")


if __name__ == "__main__":
    main()
