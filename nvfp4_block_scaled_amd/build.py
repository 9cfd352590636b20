"""Build the gfx950 HIP library libnvfp4.so in-tree with hipcc.

Each source is compiled to an object in parallel (every translation unit holds
its own device code), then the objects are linked into the shared library.

Usage: python -m nvfp4_block_scaled_amd.build   (or call build()).
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libnvfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "config.hip", "quantize.hip", "gemm_w4a4.hip", "gemm_w4a16.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",          # the quantizer's steps are single IEEE ops; keep every file the same
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))
    return res


def build(verbose=False):
    with tempfile.TemporaryDirectory(prefix="nvfp4_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC] + FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(min(len(cmds), max(1, os.cpu_count() or 1))) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
