"""Build libattn_decode.so (the C-ABI library) and libattn_probe.so (the
read-only bandwidth probes of include/attn_probe.h) in-tree with hipcc for
gfx950.

Every translation unit is compiled with hipcc; the shared object is linked
against the HIP runtime that torch loads (``torch/lib/libamdhip64.so``) so a
process that uses torch for memory and streams holds exactly one HIP runtime.
Without torch on the machine the system runtime under /opt/rocm/lib is used.

    python -m split_kv_paged_amd.build        # or __graft_entry__.build()
"""
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libattn_decode.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
PROBE_DIR = os.path.join(PKG, "probe")
PROBE_LIB_PATH = os.path.join(PKG, "libattn_probe.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # packed-FP32 instructions stay off (v_pk_fma_f32 and kin)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-lambda-capture",
]


def _hip_runtime_dir():
    """Directory of the libamdhip64.so that torch loads, else ROCm's."""
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec and spec.origin:
            d = os.path.join(os.path.dirname(spec.origin), "lib")
            if os.path.exists(os.path.join(d, "libamdhip64.so")):
                return d
    except Exception:
        pass
    return os.path.join(ROCM, "lib")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def sources():
    """Sources of libattn_decode.so."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def probe_sources():
    """Sources of libattn_probe.so."""
    return sorted(glob.glob(os.path.join(PROBE_DIR, "*.hip")))


def build(verbose=False, jobs=None):
    """Compile every source and link both libraries.  Always rebuilds."""
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc") or hipcc
    os.makedirs(BUILD_DIR, exist_ok=True)
    targets = [(LIB_PATH, sources()), (PROBE_LIB_PATH, probe_sources())]
    objs = {}
    procs = []
    for lib_path, srcs in targets:
        objs[lib_path] = []
        for src in srcs:
            obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
            cmd = [hipcc] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
            if src.endswith(".cpp"):
                cmd[1:1] = ["-x", "hip"]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((subprocess.Popen(cmd), src))
            objs[lib_path].append(obj)
    failed = [s for p, s in procs if p.wait() != 0]
    if failed:
        raise RuntimeError("hipcc failed on: " + ", ".join(failed))
    rt = _hip_runtime_dir()
    for lib_path, _ in targets:
        tmp = lib_path + ".tmp%d" % os.getpid()
        link = ["g++", "-shared", "-o", tmp] + objs[lib_path] + [
            "-L" + rt, "-l:libamdhip64.so", "-Wl,-rpath," + rt,
            "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-Wl,--no-undefined", "-lpthread"]
        _run(link, verbose)
        os.replace(tmp, lib_path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
