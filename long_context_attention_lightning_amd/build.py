"""Build liblisa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "liblisa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 VALU ops are disabled for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments (up to 16 dwords) are preloaded into
    # SGPRs at wave launch instead of being read from the argument segment
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    return err


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object (in parallel), then link the
    shared library; always rebuilds."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[hipcc, *HIPCC_FLAGS, *inc, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        errs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    errs.append(_run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]))
    err = "\n".join(e for e in errs if e.strip())
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
