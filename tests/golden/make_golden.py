"""Write the oracle regression fixture for the tiny workload (round 0).

Calls only the CPU oracle and the seeded input generator.  The pages print no
worked example of the recurrence, so this file pins the oracle to its own
earlier output: a change to the oracle's arithmetic must regenerate it, and
the commit that does so must say why.

Usage: python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from gated_delta_rule_rows_amd import synth  # noqa: E402

OUT = os.path.join(HERE, "tiny_round0.txt")
STATE_ROWS = (0, 63, 127)


def compute():
    w = synth.WORKLOADS["tiny"]
    r = synth.rows(w.seed, 0, w.L, w.T, w.H)
    s0 = np.zeros((w.L, w.H, synth.D, synth.D), np.float32)
    s, o = oracle.scan_rows(s0, r["q"], r["k"], r["v"], r["g"], r["beta"])
    return o[0, :, 0], s[0, 0, list(STATE_ROWS)]


def main():
    o, srows = compute()
    with open(OUT, "w") as f:
        f.write("# tiny workload round 0 (seed 0, L=1 H=1 T=8, zero state): oracle output\n")
        f.write("# written by tests/golden/make_golden.py; f32 words as hex\n")
        for t in range(o.shape[0]):
            f.write(f"o {t} " + " ".join(f"{w:08x}" for w in o[t].view(np.uint32)) + "\n")
        for n, i in enumerate(STATE_ROWS):
            f.write(f"s {i} " + " ".join(f"{w:08x}" for w in srows[n].view(np.uint32)) + "\n")


if __name__ == "__main__":
    main()
