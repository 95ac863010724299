"""Compile the HIP library ``libvqm.so`` for gfx950, in-tree.

``python -m full_reference_video_amd.build`` or ``build()``.  Always
recompiles.  Flags:

* ``--offload-arch=gfx950`` only (MI355X).
* ``-ffp-contract=off``: no implicit FMA contraction, so expressions that must
  round the same way for both planes (the SSIM map's mirrored numerator and
  denominator) do; the kernels ask for FMA explicitly where they want it.
* ``-fhip-fp32-correctly-rounded-divide-sqrt``: fp32 ``/`` is IEEE division
  (the ssimulacra2 pair quotients rely on correctly rounded partial
  quotients).
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32 math.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvqm.so")

SOURCES = ["vqm_runtime.cpp", "ssim_step.hip", "msssim.hip", "ss2_stats.hip", "ss2_chain.hip", "probe.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-fvisibility=hidden",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so; drop
    # that line, keep everything else.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
