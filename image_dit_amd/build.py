"""Build libditattn.so (the HIP kernels and their C ABI) for gfx950, in-tree.

Plain hipcc, ahead of time: one shared library that links the HIP runtime
and nothing else.  Device code is built with correctly rounded fp32 division
(the Sage quantizer must match IEEE division bit for bit) and without the
packed-fp32 feature.
"""
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libditattn.so")
SOURCES = ["abi.hip", "attn_bf16.hip", "attn_sage.hip", "prepare.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags():
    return ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC",
            "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-rdc",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def build(force: bool = True, verbose: bool = False, out_path: str = None, defines=()) -> str:
    """Compile every source and link libditattn.so (or `out_path`, with extra -D defines)."""
    lib_path = out_path or LIB
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    deps = srcs + [os.path.join(CSRC, "common.hpp"), os.path.join(CSRC, "launch.hpp"),
                   os.path.join(ROOT, "include", "ditattn.h")]
    if not force and os.path.exists(lib_path) and os.path.getmtime(lib_path) >= max(os.path.getmtime(d) for d in deps):
        return lib_path
    with tempfile.TemporaryDirectory(prefix="ditattn_build_") as tmp:
        objs = []
        for src in srcs:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc()] + compile_flags() + ["-D" + d for d in defines] + ["-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (src, r.stderr))
            if verbose:
                print(" ".join(cmd))
            objs.append(obj)
        out = os.path.join(tmp, "libditattn.so")
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s" % r.stderr)
        shutil.copyfile(out, lib_path + ".tmp")
        os.replace(lib_path + ".tmp", lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
