"""Build bitlinear_amd/libbitlinear.so for gfx950 with hipcc (in-tree).

Device code: -O3, no FP contraction (each fp32/fp64 multiply and add rounds on
its own, as the numerics of the ABI state), correctly rounded division and
square root (the HIP defaults), and packed-fp32 instructions disabled.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbitlinear.so")
ARCH = "gfx950"

HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wextra"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def torch_lib_dir():
    """torch's lib directory (found without importing torch). torch ships its own
    HIP runtime there; the library must link that same runtime, or a process
    that uses torch would hold two HIP runtimes whose streams and allocations do
    not know each other."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("torch is not importable: the library links torch's HIP runtime")
    lib = os.path.join(list(spec.submodule_search_locations)[0], "lib")
    if not os.path.exists(os.path.join(lib, "libamdhip64.so")):
        raise RuntimeError(f"no libamdhip64.so under {lib}")
    return lib


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src, verbose):
    out = os.path.join(BUILD, src + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [_hipcc(), *HIP_FLAGS, "-c", path, "-o", out]
    else:
        cmd = ["g++", *HOST_FLAGS, "-c", path, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise
    noise = ("packed-fp32-ops", "is not a recognized feature")
    warn = "\n".join(l for l in r.stderr.splitlines() if l.strip() and not any(s in l for s in noise))
    if warn and verbose:
        print(warn, flush=True)
    return out


def build(verbose=True, jobs=8):
    """Compile every source under csrc/ and link libbitlinear.so. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources()))
    tmp = LIB + ".tmp"
    tl = torch_lib_dir()
    cmd = ["g++", "-shared", "-fPIC", *objs, "-o", tmp, "-L" + tl, "-l:libamdhip64.so", "-Wl,-rpath," + tl,
           "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
