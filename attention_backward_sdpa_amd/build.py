"""Build the HIP library in-tree: attention_backward_sdpa_amd/libsdpa_bwd.so for gfx950.

    python -m attention_backward_sdpa_amd.build      (or call build())
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "sdpa_bwd.hip")
OUT = os.path.join(HERE, "libsdpa_bwd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    # the LDS-DMA loads are inline assembly that sets M0; clang warns that M0 is a reserved
    # register (tests/test_isa.py checks that nothing else in the kernels uses it)
    "-Wno-inline-asm",
]


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles); returns the path of the shared object."""
    tmp = OUT + ".tmp"
    cmd = [HIPCC, *FLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, OUT)
    return OUT


def device_assembly() -> str:
    """The gfx950 assembly of the library's kernels (device pass only), for inspection."""
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "--offload-device-only",
           "-S", SRC, "-o", "-"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    return res.stdout


if __name__ == "__main__":
    print(build(verbose=True))
