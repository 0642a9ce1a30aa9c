"""Build libmeswish.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("meswish.hip", "dense_bn.hip", "fft_conv.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libmeswish.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # No packed-fp32 instructions (v_pk_*_f32) anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


# A test build of the activation kernels alone with three tiles per launch,
# so that the split of long tensors into several launches runs on tensors
# small enough for a GPU test (the library's own limit is 2^30 tiles).
SPLIT_TEST_LIBRARY = os.path.join(HERE, "libmeswish_split3.so")
SPLIT_TEST_TILES = 3
# What that build exports: the activation entry points and their helpers.
SPLIT_TEST_NAMES = ("swish_fwd", "swish_bwd", "swish_fwd_grouped", "swish_bwd_grouped",
                    "meswish_act_fwd", "meswish_act_bwd", "meswish_strerror",
                    "meswish_version", "meswish_copy", "meswish_plan")


def build(output: str = LIBRARY, extra_flags: list[str] | None = None,
          sources: list[str] | None = None) -> str:
    """Compile libmeswish.so (always recompiles) and return its path."""
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", *(sources or SOURCES),
           "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def build_split_test() -> str:
    """The test build of the activation kernels with SPLIT_TEST_TILES tiles
    per launch (used by the GPU tests of the multi-launch split only)."""
    return build(SPLIT_TEST_LIBRARY, [f"-DMESWISH_MAX_LAUNCH_TILES={SPLIT_TEST_TILES}"],
                 [os.path.join(HERE, "csrc", "meswish.hip")])


if __name__ == "__main__":
    print(build())
