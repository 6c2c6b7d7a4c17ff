"""Build the test-support library ``tests/hip/libnvfp4_test_support.so`` (gfx950).

It holds kernels that run the library's device code for encoding and
dequantization over inputs the converter tests choose; the tests compare
every output with the CPU oracle.  Called by ``__graft_entry__.build()``.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libnvfp4_test_support.so")


def build(verbose: bool = False) -> str:
    sys.path.insert(0, ROOT)
    from nvfp4_w4a16_lm_amd import build_lib

    tmp = LIB + ".tmp"
    cmd = [build_lib.hipcc(), *build_lib.COMMON_FLAGS, "-I", os.path.join(ROOT, "nvfp4_w4a16_lm_amd", "csrc"),
           "-shared", "-x", "hip", os.path.join(HERE, "converter_sweep.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"test-support build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
