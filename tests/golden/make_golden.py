"""Writes tests/golden/exact_tiny.json from the exact rational evaluation in
oracle/exact.py (and nothing else).

The pages print no numeric example of the recurrence, so the golden values are
computed without any rounding: inputs are dyadic rationals (exact in fp32), the
gate is stored as an fp32 log value g and its retention a = exp(g) is taken as
the exact rational value of the nearest double, and the recurrence
S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t is then
run in Fraction arithmetic.  Two cases: dk != dv (catches transposed operands)
and a nonzero starting state.
"""
import json
import math
import os
import sys
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle import exact  # noqa: E402


def _dyadic(rng, shape, den=16, lo=-16, hi=16):
    return (rng.integers(lo, hi + 1, size=shape) / den).astype(np.float32)


def case(seed, T, dk, dv, with_state):
    rng = np.random.default_rng(seed)
    q = _dyadic(rng, (T, dk))
    k = _dyadic(rng, (T, dk), den=8, lo=-6, hi=6)
    v = _dyadic(rng, (T, dv))
    g = np.array([0.0, -0.25, -1.0, -0.0625, -2.5, -0.5][:T], dtype=np.float32)
    beta = np.array([0.5, 0.25, 1.0, 0.375, 0.75, 0.125][:T], dtype=np.float32)
    S0 = _dyadic(rng, (dv, dk)) if with_state else None
    F = lambda x: Fraction(float(x))  # noqa: E731  exact: fp32 -> double -> rational
    a = [Fraction(math.exp(float(x))) for x in g]
    o, S = exact.scan([[F(x) for x in r] for r in q], [[F(x) for x in r] for r in k],
                      [[F(x) for x in r] for r in v], a, [F(x) for x in beta],
                      None if S0 is None else [[F(x) for x in r] for r in S0])
    return dict(T=T, dk=dk, dv=dv, q=q.tolist(), k=k.tolist(), v=v.tolist(), g=g.tolist(),
                beta=beta.tolist(), state_in=None if S0 is None else S0.tolist(),
                o=[[float(x) for x in r] for r in o], state_out=[[float(x) for x in r] for r in S],
                o_exact=[[str(x) for x in r] for r in o])


def main():
    cases = [case(1, 5, 3, 2, False), case(2, 6, 4, 5, True)]
    doc = dict(source="oracle/exact.py via tests/golden/make_golden.py (exact rational "
                      "arithmetic; the pages print no worked example)",
               cases=cases)
    with open(os.path.join(HERE, "exact_tiny.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
