"""Build libmoe_nvfp4.so in-tree with hipcc for gfx950."""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_nvfp4.so")
# profiling build: the persistent kernels record per-block phase timestamps (-DMOE_TIMELINE)
TIMELINE_BUILD = os.path.join(PKG, "_build_timeline")
TIMELINE_LIB = os.path.join(PKG, "libmoe_nvfp4_timeline.so")
SOURCES = ["api.hip", "route.hip", "group.hip", "ffn.hip", "combine.hip", "pack.hip", "gemm.hip",
           "layer_small.hip", "combine_norm.hip", "mx8.hip", "route_group.hip"]
HEADERS = [os.path.join(CSRC, h) for h in ("common.h", "dot.h", "sync.h", "group_dev.h", "select_dev.h")] + [
    os.path.join(ROOT, "include", "moe_nvfp4.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # keep fp32 arithmetic in scalar form (no packed fp32 VALU instructions)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(src, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, src + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose=True, timeline=False):
    """Compile every HIP source (always, also when a library exists) and link the library.
    timeline=True builds the profiling library (libmoe_nvfp4_timeline.so, -DMOE_TIMELINE)."""
    bdir, lib = (TIMELINE_BUILD, TIMELINE_LIB) if timeline else (BUILD, LIB)
    extra = ("-DMOE_TIMELINE",) if timeline else ()
    os.makedirs(bdir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, bdir, extra), SOURCES))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib, file=sys.stderr)
    return lib


if __name__ == "__main__":
    build(timeline="--timeline" in sys.argv[1:])
