"""Readers for the hand-derived fixtures under tests/golden/ (no arithmetic of the layer)."""
import math
import os
import re
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def frac(tok):
    return Fraction(tok)


def value(expr):
    """Evaluate a fixture value: a sum of terms; a term is a product of factors 'p/q',
    'lnN' (natural log of N) or 'p@s' (p / sqrt(s))."""
    expr = expr.strip()
    total = 0.0
    for term in re.findall(r"[+-]?[^+-]+", expr):
        sign = -1.0 if term.startswith("-") else 1.0
        term = term.lstrip("+-")
        v = 1.0
        for f in term.split("*"):
            if f.startswith("ln"):
                v *= math.log(float(Fraction(f[2:])))
            elif "@" in f:
                p, s = f.split("@")
                v *= float(Fraction(p)) / math.sqrt(float(Fraction(s)))
            else:
                v *= float(Fraction(f))
        total += sign * v
    return total
