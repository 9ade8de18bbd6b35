"""Build libppx.so (HIP for gfx950) in place.

Every HIP/C++ source under csrc/ is compiled with hipcc for gfx950 only and
linked into prompt_prefill_cross_amd/libppx.so.  Packed fp32 VALU ops are
disabled for the device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libppx.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in VGPRs: avoids per-iteration AGPR<->VGPR copies of
          # the accumulator tiles in the GEMM and attention loops
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-I", os.path.join(HERE, "..", "include")]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *CFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


# ---- host-side sanitizer build of the file parsers (CPU only) ----------------
# The host code of every source is compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer (the device code is built as usual and never
# launched by the driver) and
# linked with fuzz/fuzz_host.cpp into a driver that feeds mutated containers
# and snapshots to the parsers.  Each -fsanitize= flag is scoped to the host
# compiler with -Xarch_host.
SAN_BUILD = os.path.join(HERE, "_build_san")
FUZZ_SRC = os.path.join(HERE, "fuzz", "fuzz_host.cpp")
FUZZ_EXE = os.path.join(SAN_BUILD, "fuzz_host")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_fuzz(verbose=True):
    os.makedirs(SAN_BUILD, exist_ok=True)
    srcs = [os.path.join(CSRC, f) for f in sources()] + [FUZZ_SRC]
    newest = max(os.path.getmtime(x) for x in srcs + [os.path.join(HERE, "..", "include", "ppx.h"), __file__])
    if os.path.exists(FUZZ_EXE) and os.path.getmtime(FUZZ_EXE) >= newest:
        return FUZZ_EXE
    flags = ["-O1", "-g", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-I", os.path.join(HERE, "..", "include"), *SAN]

    def one(src):
        obj = os.path.join(SAN_BUILD, os.path.basename(src) + ".o")
        dev = [f"--offload-arch={ARCH}"] if src != FUZZ_SRC else ["--offload-host-only"]
        r = subprocess.run([HIPCC, "-x", "hip", *dev, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (host, sanitizers) failed for {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, srcs))
    tmp = FUZZ_EXE + f".tmp{os.getpid()}"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", *SAN, "-o", tmp, *objs, "-lpthread"], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (host, sanitizers) failed:\n{r.stderr}")
    os.replace(tmp, FUZZ_EXE)
    if verbose:
        print(f"built {FUZZ_EXE}")
    return FUZZ_EXE


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "fuzz":
        build_fuzz()
    else:
        build()
    sys.exit(0)
