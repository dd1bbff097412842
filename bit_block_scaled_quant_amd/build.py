"""Build libnvfp4.so (HIP, gfx950) in-tree with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC_DIR = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "quantize.hip", "dequantize.hip", "gemm.hip", "mx.hip"]
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every fp32 step of the quantizer is a separately rounded operation
    "-ffp-contract=off",
    # no packed-fp32 instructions (v_pk_*_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(verbose=False):
    srcs = [os.path.join(SRC_DIR, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB_PATH)
    return r.stderr


if __name__ == "__main__":
    print(build(verbose=True))
