"""Input generator checks (no GPU): the planted family with c = 1 on every
head is the planted recipe with the multiplier fixed, and shares every other
draw with the planted family."""
import numpy as np

from synth import WORKLOADS, prefill_inputs, to_f64
from synth.planted import sharpness


def test_planted_c1_equals_planted_where_c_is_one():
    w = WORKLOADS["tiny"]  # its multiplier range is [1, 1]
    assert w.sharp_lo == w.sharp_hi == 1.0
    a = prefill_inputs(w, family="planted", L=300)
    b = prefill_inputs(w, family="planted_c1", L=300)
    for n in ("q", "k", "v", "do"):
        assert np.array_equal(a[n], b[n]), n


def test_planted_c1_fixes_only_the_multiplier():
    w = WORKLOADS["sweep32k"]
    heads = [0, 1, 2]
    a = prefill_inputs(w, family="planted", L=520, heads=heads)
    b = prefill_inputs(w, family="planted_c1", L=520, heads=heads)
    for n in ("k", "v", "do"):
        assert np.array_equal(a[n], b[n]), n
    cs = [sharpness(w, 0, h) for h in heads]
    assert max(abs(c - 1.0) for c in cs) > 0.05  # the planted heads really are rescaled
    for h, c in zip(heads, cs):
        q1 = to_f64(b["q"][0, h], "bf16")
        qc = to_f64(a["q"][0, h], "bf16")
        # both are the same fp64 query (times c, times 1) rounded once to bf16
        # (unit roundoff 2^-8): |qc - c q1| <= 2^-8 (|c x| + c |x|), |x| <= |q1| / (1 - 2^-8)
        bound = 2.0 ** -7 * c * np.abs(q1) / (1 - 2.0 ** -8) + 1e-300
        assert np.all(np.abs(qc - c * q1) <= bound), h
