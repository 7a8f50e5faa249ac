"""Build libmoe4.so (HIP, gfx950) in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object in parallel, then linked
into bit_mixture_experts_amd/libmoe4.so. No -ffast-math: the NF4 quantiser
relies on IEEE fp32 division.

build_asan() also links libmoe4_asan.so: the same library with the C entry
points (moe4_abi.hip) compiled with AddressSanitizer on their host code. It
exists to run the argument validation of the C ABI under ASan on a machine
without a GPU (tests/test_abi_asan.py); nothing else loads it.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe4.so")
LIB_ASAN = os.path.join(HERE, "libmoe4_asan.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # keep the compiler from emitting packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, obj, extra):
    cmd = [hipcc(), *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{r.stderr}")
    return obj


def build(verbose=False, extra=()):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    objs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s),
                          os.path.join(BUILD, s[:-4] + ".o"), list(extra)) for s in srcs]
        for f in futs:
            objs.append(f.result())
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# AddressSanitizer on the host pass only (each -fsanitize= goes to the host)
ASAN_FLAGS = "-g -Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def build_asan(verbose=False):
    """libmoe4_asan.so: moe4_abi.hip (the C entry points and their argument
    validation) recompiled with AddressSanitizer on its host code, linked with
    the other objects of the last build(); the ASan runtime is left undefined
    and comes from LD_PRELOAD at run time."""
    out_dir = os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = []
    for s in srcs:
        if s == "moe4_abi.hip":
            continue
        obj = os.path.join(BUILD, s[:-4] + ".o")
        if not os.path.exists(obj):
            raise RuntimeError(f"{obj} is missing: run build() first")
        objs.append(obj)
    objs.append(_compile(os.path.join(CSRC, "moe4_abi.hip"), os.path.join(out_dir, "moe4_abi.o"),
                         ASAN_FLAGS))
    tmp = LIB_ASAN + ".tmp"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"ASan link failed:\n{r.stderr}")
    os.replace(tmp, LIB_ASAN)
    if verbose:
        print(f"built {LIB_ASAN}")
    return LIB_ASAN


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
