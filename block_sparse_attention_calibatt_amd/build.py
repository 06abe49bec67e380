"""Build libcalibatt.so (gfx950) in-tree with hipcc, and the matrix-core
rate probe (`mfma_rate`, run by bench.py for the roofline).

Usage: python -m block_sparse_attention_calibatt_amd.build [--verbose]
"""

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcalibatt.so")
PROBE_SRC = os.path.join(CSRC, "probes", "mfma_rate.hip")
PROBE = os.path.join(PKG, "mfma_rate")
SOURCES = ["api.hip", "attn_fwd.hip", "mass.hip", "compile.hip", "share.hip", "intervals.hip", "repeat.hip"]
ARCH = os.environ.get("CALIBATT_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 ops stay off: the kernels are written for plain fp32 VALU
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every atomic here is issued by one lane (queue pops); the atomic
    # optimizer would turn each into a wave scan that waits for the atomic's
    # return on the spot
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


# The attention and calibration kernels keep their matrix-core accumulators
# in ordinary vector registers (mixing in accumulation registers splits the
# register file in half at two waves per SIMD and spills, and every score
# the vector units read would first be copied out), which needs the
# vector-register form of the matrix instructions.
PER_FILE_FLAGS = {f: ["-mllvm", "--amdgpu-mfma-vgpr-form"] for f in ("attn_fwd.hip", "mass.hip", "repeat.hip")}


def build(verbose=False, extra=()):
    """Compile every source to an object (in parallel), then link the library."""
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="calibatt_build_") as tdir:
        def compile_one(src):
            obj = os.path.join(tdir, src + ".o")
            flags = [f for f in FLAGS if f != "-shared"]
            cmd = [hipcc()] + flags + PER_FILE_FLAGS.get(src, []) + list(extra) + [
                "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            return src, obj, res

        def build_probe():
            flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
            cmd = [hipcc()] + flags + ["-mllvm", "--amdgpu-mfma-vgpr-form", PROBE_SRC, "-o", PROBE + ".tmp"]
            if verbose:
                print(" ".join(cmd), flush=True)
            return subprocess.run(cmd, capture_output=True, text=True)

        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
            probe = ex.submit(build_probe)
            results = list(ex.map(compile_one, SOURCES))
            pres = probe.result()
        if pres.returncode != 0:
            sys.stderr.write(pres.stdout + pres.stderr)
            raise RuntimeError(f"hipcc failed on {PROBE_SRC} with exit code {pres.returncode}")
        os.replace(PROBE + ".tmp", PROBE)
        for src, _, res in results:
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed on {src} with exit code {res.returncode}")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + [o for _, o, _ in results] + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"linking failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
