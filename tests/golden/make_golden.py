"""Writes the stored expected values under tests/golden/ from the oracle only.

    python tests/golden/make_golden.py

nf4_codebook.txt: the 16 codes of the normal-quantile table (tail probability
0.9677083), rounded to bfloat16, as hex floats.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def main():
    cb, unr = oracle.codebook()
    with open(os.path.join(HERE, "nf4_codebook.txt"), "w") as f:
        f.write("# NF4-style codebook: normal quantiles normalised to [-1, 1] with an exact\n")
        f.write("# zero, tail probability %r, each rounded to the nearest bfloat16.\n" % oracle.DELTA)
        f.write("# Written by tests/golden/make_golden.py from the oracle; one code per line.\n")
        for i, (c, u) in enumerate(zip(cb, unr)):
            f.write("%-24s # c[%2d] = %.9g (unrounded %.17g)\n" % (float(c).hex(), i, c, u))


if __name__ == "__main__":
    main()
