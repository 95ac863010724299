"""Write tests/golden/oracle_scores.json from the oracle alone.

Regression record of the oracle's own outputs on the seeded frames: a later
change to the oracle's arithmetic shows up as a mismatch here and must name
the passage that justifies it.  Calls nothing but ``oracle`` and the input
generator.  Run from the repository root: ``python tests/golden/make_golden.py``.
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from full_reference_video_amd import synth  # noqa: E402

FRAMES = [0, 1, 17]


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


if __name__ == "__main__":
    main()
