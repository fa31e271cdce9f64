"""Build the HIP library positions_aware_cached_amd/libmllm.so for gfx950.

hipcc compiles the host layer (csrc/mllm.cpp) and the kernels (csrc/*.hip)
into one shared library that exports the C ABI of include/mllm.h.  Packed
FP32 instruction selection is switched off for device code; nothing is built
with fast-math or denormal flushing.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmllm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")) + glob.glob(os.path.join(CSRC, "*.hip")))


PROBE_SRC = os.path.join(HERE, "probe", "read_ceiling.hip")
PROBE_LIB = os.path.join(HERE, "libreadprobe.so")
# diagnosis build: the same library with the decode kernel's per-group wall-clock
# stamps compiled in (MLLM_STAMPS; read back with mllm_debug_stamps), loaded only
# by `bench.py --phases`
STAMPS_LIB = os.path.join(HERE, "libmllm_stamps.so")


def build(out=LIB, verbose=False, jobs=8):
    """Compile every source (in parallel) and link out; also the read-ceiling
    probe library that bench.py loads (measurement code, a library of its
    own).  Returns out."""
    srcs = sources()
    tmpdir = tempfile.mkdtemp(prefix="mllm_build_")
    try:
        res = _build_in(srcs, tmpdir, out, verbose, jobs)
        if out == LIB:
            _build_in([PROBE_SRC], tmpdir, PROBE_LIB, verbose, jobs)
        return res
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)


def _build_in(srcs, tmpdir, out, verbose, jobs):
    procs, objs = [], []
    for s in srcs:
        obj = os.path.join(tmpdir, os.path.basename(s) + ".o")
        cmd = [HIPCC, *COMMON, "-c", s, "-o", obj]
        if s.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd))
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs)
            procs = []
    _wait(procs)
    tmp = out + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, out)
    return out


def _wait(procs):
    failed = []
    for s, p in procs:
        outp, _ = p.communicate()
        text = "\n".join(l for l in outp.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((s, text))
        elif text.strip():
            sys.stderr.write(text + "\n")
    if failed:
        for s, text in failed:
            sys.stderr.write(f"--- {s}\n{text}\n")
        raise RuntimeError("HIP build failed: " + ", ".join(os.path.basename(s) for s, _ in failed))


def build_stamps(verbose=False, jobs=8):
    """The library with MLLM_STAMPS defined, as STAMPS_LIB."""
    global COMMON
    saved = COMMON
    COMMON = COMMON + ["-DMLLM_STAMPS"]
    tmpdir = tempfile.mkdtemp(prefix="mllm_build_")
    try:
        return _build_in(sources(), tmpdir, STAMPS_LIB, verbose, jobs)
    finally:
        COMMON = saved
        shutil.rmtree(tmpdir, ignore_errors=True)


if __name__ == "__main__":
    if "--stamps" in sys.argv:
        print(build_stamps(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
