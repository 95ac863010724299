"""Write tests/golden/oracle_scores.json and msssim_2160p8_oracle.json from
the oracle alone.

oracle_scores.json is the regression record of the oracle's own outputs on
the seeded frames: a later change to the oracle's arithmetic shows up as a
mismatch here and must name the passage that justifies it.
msssim_2160p8_oracle.json holds the oracle's score and 15 level means for
every frame of the 3840x2160 8-bit MS-SSIM workload (seconds per frame on one
core, so it is computed here, in parallel processes, once), for the GPU test
that compares every frame.  Calls nothing but ``oracle`` and the input
generator.  Run from the repository root: ``python tests/golden/make_golden.py``.
"""

import json
import multiprocessing
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from full_reference_video_amd import synth  # noqa: E402

FRAMES = [0, 1, 17]


def _msssim_frame(t):
    src = synth.FrameSource(5)
    score, lcs = oracle.msssim(*src.pair(t), src.bpc, want_lcs=True)
    return t, score, lcs.tolist()


def write_msssim_workload(processes=None):
    src = synth.FrameSource(5)
    n = src.workload.frames
    with multiprocessing.get_context("fork").Pool(processes or min(8, os.cpu_count() or 1)) as pool:
        rows = sorted(pool.map(_msssim_frame, range(n)))
    out = {"_about": "oracle MS-SSIM score and level means (L1..L5, C1..C5, S1..S5) of every frame of the "
                     "3840x2160 8-bit MS-SSIM workload (synth.FrameSource(5)); written by make_golden.py",
           "workload": src.workload.name, "w": src.w, "h": src.h, "bpc": src.bpc,
           "frames": {str(t): {"score": score, "lcs": lcs} for t, score, lcs in rows}}
    path = os.path.join(ROOT, "tests", "golden", "msssim_2160p8_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)


def main():
    out = {"_about": "oracle outputs on the seeded frames; written by make_golden.py",
           "float_ssim": {}, "ms_ssim": {}}
    for c in (1, 2, 3, 4):
        src = synth.FrameSource(c)
        frames = [t for t in FRAMES if t < src.workload.frames]
        out["float_ssim"][str(c)] = {str(t): oracle.ssim(*src.pair(t), src.bpc) for t in frames}
    src = synth.FrameSource(5)
    score, lcs = oracle.msssim(*src.pair(0), 8, want_lcs=True)
    out["ms_ssim"]["5"] = {"0": {"score": score, "lcs": lcs.tolist()}}
    small = synth.FrameSource(5, w=640, h=360)
    score, lcs = oracle.msssim(*small.pair(1), 8, want_lcs=True)
    out["ms_ssim"]["5@640x360"] = {"1": {"score": score, "lcs": lcs.tolist()}}
    path = os.path.join(ROOT, "tests", "golden", "oracle_scores.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)
    write_msssim_workload()


if __name__ == "__main__":
    main()
