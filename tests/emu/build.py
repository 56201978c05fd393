"""Build tests/emu/_build/libep_emu.so: the library's own HIP sources compiled
for the host CPU against a small emulation of the HIP device API (lane fibers,
wave rendezvous, workgroup barriers; see fake/hip/hip_runtime.h).

Test infrastructure only.  It lets the CPU test suite run the real kernel code
-- the fused persistent mode included -- against the CPU oracle, with a limited
number of co-resident workgroups."""
import concurrent.futures as cf
import fcntl
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "combine_ep_route_topk_amd", "csrc")
OUT = os.path.join(HERE, "_build")
LIB = os.path.join(OUT, "libep_emu.so")


def compiler():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++"),
              shutil.which("clang++") or ""):
        if c and os.path.exists(c):
            return c
    return None


def _inputs():
    return (glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h")) +
            glob.glob(os.path.join(HERE, "fake", "**", "*"), recursive=True) +
            [os.path.join(HERE, "emu_runtime.cpp"), os.path.abspath(__file__)])


def build(extra=(), variant=None):
    """Builds the library unless it is newer than every input.  `variant`
    names a separate build (its own objects and library file) compiled with
    the `extra` flags -- the emulation's negative controls use this.
    Concurrent callers -- parallel test workers -- take turns on a lock file,
    so none links another's half-written objects."""
    cxx = compiler()
    if cxx is None:
        raise RuntimeError("clang++ not found")
    out = OUT if variant is None else os.path.join(OUT, variant)
    lib = LIB if variant is None else os.path.join(OUT, f"libep_emu_{variant}.so")
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(OUT, ".lock"), "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        if os.path.exists(lib) and \
                os.path.getmtime(lib) >= max(os.path.getmtime(f) for f in _inputs()):
            return lib
        return _build(cxx, extra, out, lib)


def _build(cxx, extra, out, lib):
    flags = ["-std=c++17", "-O1", "-g", "-fPIC",
             "-I", os.path.join(HERE, "fake"), "-I", os.path.join(ROOT, "include"), *extra]
    jobs = [(os.path.join(CSRC, f), os.path.join(out, f + ".o"), True)
            for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")]
    jobs.append((os.path.join(HERE, "emu_runtime.cpp"), os.path.join(out, "emu_runtime.o"), False))

    def one(job):
        src, obj, as_cxx = job
        cmd = [cxx, *flags] + (["-x", "c++"] if as_cxx else []) + ["-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode:
            raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(one, jobs))
    subprocess.run([cxx, "-shared", "-o", lib + ".tmp", *objs, "-lpthread", *extra], check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build())
