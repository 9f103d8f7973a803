"""Build liblazyattn.so for gfx950 with hipcc (sources under csrc/, ABI in include/)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblazyattn.so")
SOURCES = ["api.hip", "plan.hip", "decode.hip", "mixed.hip", "materialize.hip", "probe.hip", "ingest.hip", "pool.cpp", "share.cpp", "host.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall",
         "-Wno-unused-result", "-Wno-unused-variable",
         # packed fp32 VALU ops are disabled for every HIP source of this library
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src, extra):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    objs = []
    for src, obj, r in results:
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        if verbose or resource_usage:
            sys.stderr.write("".join(line + "\n" for line in (r.stdout + r.stderr).splitlines()
                                     if "warning: ignoring" not in line and
                                     "packed-fp32-ops" not in line))
        objs.append(obj)
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, resource_usage="--usage" in sys.argv))
