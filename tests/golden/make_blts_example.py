"""Writes the stand-in patcher's boundaries for tests/golden/blts_targets_example.json.

Calls only the oracle's patcher (the published SplitMix64 rule).  The rest of
the fixture (targets, accept lengths, appended bytes, pass counts) is worked
by hand from these boundaries; see the fixture's "derivation" field.

  python tests/golden/make_blts_example.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import patcher  # noqa: E402

PATH = os.path.join(HERE, "blts_targets_example.json")

if __name__ == "__main__":
    g = json.load(open(PATH))
    full = g["prompt"] + g["continuation"] + g["extension"]
    patch, ends = patcher.segment(full, g["prompt_patches"], g["salt"])
    g["patch_ends"] = [int(i) for i in range(len(full)) if ends[i]]
    with open(PATH, "w") as f:
        json.dump(g, f, indent=1)
        f.write("\n")
    print(g["patch_ends"])
