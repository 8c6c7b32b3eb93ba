"""Writes the stored expected values under tests/golden/ from the oracle only.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def main():
    n = oracle.skipped_closed_form(256, 64, 1e4, 1.0)
    with open(os.path.join(HERE, "count_s256_d64.txt"), "w") as f:
        f.write("# Dropped (query, key, pair) terms per head, causal prefill, S=256, d=64,\n")
        f.write("# RoPE base 1e4, alpha=1 (the fp32 parity workload).  Written by\n")
        f.write("# tests/golden/make_golden.py from the oracle's closed form; the CPU tests\n")
        f.write("# also re-derive it by brute-force enumeration of every (i, j, p).\n")
        f.write("%d\n" % n)
    print(n)


if __name__ == "__main__":
    main()
