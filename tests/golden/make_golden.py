"""Writes tests/golden/single_layer_snapshot.txt from the CPU oracle only.

Run from the repository root:  python tests/golden/make_golden.py
The snapshot pins the oracle's outputs on the 4096x4096 single-layer workload
(the xorshift draws of the page "Weight quantization", section "Code") so that
an unintended change to the oracle shows up as a test failure.
"""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

ROWS = [0, 1, 2, 1000, 2047, 4095]


def main():
    w, x = synth.page_single_layer(4096, 4096)
    p, s16, z = oracle.quantize_ref(w[ROWS])
    y = oracle.gemv_ref(p, s16, z, x)[0]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "single_layer_snapshot.txt")
    with open(out, "w") as fh:
        fh.write("# Written by tests/golden/make_golden.py from oracle/ only (CPU).\n")
        fh.write("# Workload: W 4096x4096 = 0.02*U(-1,1), x 1x4096 = U(-1,1), xorshift draws.\n")
        fh.write("rows = " + " ".join(str(r) for r in ROWS) + "\n")
        for i, r in enumerate(ROWS):
            fh.write(f"packed_head_{r} = {bytes(p[i][:32]).hex()}\n")
            fh.write(f"s16_head_{r} = " + " ".join(f"{v:04x}" for v in s16.view(np.uint16)[i][:8]) + "\n")
            fh.write(f"zero_head_{r} = " + " ".join(str(v) for v in z[i][:8]) + "\n")
            fh.write(f"y_{r} = {float(y[i]).hex()}\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
