"""Build the HIP library in-tree: attention_backward_sdpa_amd/libsdpa_bwd.so for gfx950.

    python -m attention_backward_sdpa_amd.build      (or call build())
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "sdpa_bwd.hip")
# translation units: the host side with the small kernels, and the main kernel's instantiations
# of each kernel head dim (the bulk of the compile time), built in parallel
SOURCES = [SRC] + [os.path.join(HERE, "csrc", f"main_d{d}.hip") for d in (32, 64, 128, 192, 256)] + \
    [os.path.join(HERE, "csrc", f"main_ilp_d{d}.hip") for d in (128, 256)]
# per-source flags: main_ilp_d*.hip hold the main-kernel instantiations that run faster under the
# backend's latency-oriented scheduler (see IlpSched in main_launch.h)
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
SOURCE_FLAGS = {"main_ilp_d128.hip": _ILP, "main_ilp_d256.hip": _ILP}


def _src_flags(src):
    return SOURCE_FLAGS.get(os.path.basename(src), [])
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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    return res.stdout


def _parallel(cmds, verbose):
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda c: _run(c, verbose), cmds))


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles); returns the path of the shared object."""
    compile_flags = [f for f in FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="sdpa_bwd_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        _parallel([[HIPCC, *compile_flags, *_src_flags(src), "-c", src, "-o", obj]
                   for src, obj in zip(SOURCES, objs)], verbose)
        tmp = OUT + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, OUT)
    return OUT


def device_assembly() -> str:
    """The gfx950 assembly of the library's kernels (device pass only), for inspection."""
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    return "\n".join(_parallel([[HIPCC, *flags, *_src_flags(src), "--offload-device-only", "-S", src,
                                 "-o", "-"] for src in SOURCES], False))


if __name__ == "__main__":
    print(build(verbose=True))
