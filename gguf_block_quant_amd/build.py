"""Build libgq.so (HIP, gfx950) in-tree with hipcc.

    python -m gguf_block_quant_amd.build

Every source under csrc/ is compiled for gfx950 only, with packed-fp32 ops
disabled and no fast-math, then linked into gguf_block_quant_amd/libgq.so.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgq.so")
BENCH_LIB = os.path.join(HERE, "libgq_bench.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Fixed code-generation contract: gfx950 only, -O3, FMA contraction on
# (only ever fuses a*b+c into one correctly rounded FMA), no fast-math, IEEE
# fp32 division, and no packed-fp32 VALU instructions.
COMPILE_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=fast",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False) -> str:
    """Compile every source and link libgq.so. Always rebuilds."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *COMPILE_FLAGS, *lang, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 target feature; that
        # warning is expected and harmless.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            print(text, file=sys.stderr)
        elif lines and verbose:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    build_bench_helpers()
    return LIB


def build_bench_helpers() -> str:
    """libgq_bench.so: measurement kernels the benchmark uses beside libgq
    (the read-stream ceiling); not part of the library's API."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "bench", "*.hip")))
    tmp = BENCH_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, *COMPILE_FLAGS, "-shared", "-o", tmp, *srcs],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    os.replace(tmp, BENCH_LIB)
    return BENCH_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
