"""Build the GPU test helpers in this folder (``libquotient_check.so``) for
gfx950, with the library's own compiler flags.  Called by
``__graft_entry__.build()``; the GPU test that loads it fails if it is
missing."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libquotient_check.so")


def build() -> str:
    from fp8_w8a8_dynamic_amd.build import ARCH, COMMON_FLAGS, hipcc
    cmd = [hipcc(), *COMMON_FLAGS, "-shared", "-x", "hip",
           os.path.join(HERE, "quotient_check.hip"), "-o", LIB + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(LIB + ".tmp", LIB)
    assert ARCH == "gfx950"
    return LIB


if __name__ == "__main__":
    print(build())
