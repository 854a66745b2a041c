"""Readers for the text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln.split()


def e2m1_table():
    return {int(c): float(v) for c, v in lines("ocp_fp4_e2m1_values.txt")}
