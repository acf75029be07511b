"""Write the stored expected streams under tests/golden/.

Calls only the oracle (and the seeded input generators).  Run from the repo
root: python tests/golden/make_golden.py
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import codebooks as cbm  # noqa: E402
from oracle import stats, stream  # noqa: E402


def main():
    seed, n, calib_seed, calib_n, chunk = 0, 1000, 1, 4096, 512
    x = synth.draw("normal", seed, n)
    cb = cbm.qlc_codebook(stats.histogram(synth.draw("normal", calib_seed, calib_n)))
    s = stream.encode_stream(x, cb, chunk)
    with open(os.path.join(HERE, "qlc_tiny_stream.hex"), "w") as f:
        f.write("# seed=%d n=%d calib_seed=%d calib_n=%d chunk=%d\n" % (seed, n, calib_seed, calib_n, chunk))
        h = s.hex()
        for i in range(0, len(h), 64):
            f.write(h[i:i + 64] + "\n")


if __name__ == "__main__":
    main()
