"""Host logic of bench.py's measurements (no GPU): the matched-work policies.

The decisions come from the oracle's forward on a small planted instance;
what is checked is the policy bookkeeping itself:
- the reference-mass policy is the optimum of total omitted mass at its tile
  count, so it can never omit more than MALA's decisions at the same count;
- every policy's per-row omitted mass and slots agree with a direct count;
- a policy that keeps every legal tile omits nothing and reproduces exact
  attention;
- the position-only window is the one whose tile count is closest to the
  target.
"""
import numpy as np
import pytest

import bench
import oracle
from synth import WORKLOADS, prefill_inputs, to_f64


@pytest.fixture(scope="module")
def case():
    w = WORKLOADS["mw8k"]
    x = prefill_inputs(w, L=1280, heads=[0, 1, 2])
    q, k, v = (to_f64(x[n][:, [0, 1, 2]], "bf16") for n in ("q", "k", "v"))
    _, _, keep, _ = oracle.fwd(q, k, v, 1.0, 128, 64)
    return w, q[0], k[0], v[0], keep[0]


def test_reference_mass_never_omits_more_than_mala(case):
    w, q, k, v, keep = case
    blocks = [0, 3, 6, 9]
    L = q.shape[1]
    for h in range(q.shape[0]):
        r = bench.policy_fidelity(q[h], k[h], v[h], keep[h], blocks, 128, 64, 1 / np.sqrt(128), window=2)
        assert r["reference_mass"]["tiles"] == r["mala"]["tiles"]
        assert r["reference_mass"]["omitted"].sum() <= r["mala"]["omitted"].sum() + 1e-12
        nrows = sum(min(b * 128 + 128, L) - b * 128 for b in blocks)
        for name in r:
            assert r[name]["omitted"].shape == (nrows,)
            assert (r[name]["omitted"] >= -1e-12).all() and (r[name]["omitted"] <= 1 + 1e-12).all()


def test_policy_counts_match_direct_count(case):
    w, q, k, v, keep = case
    L = q.shape[1]
    blocks = [2, 9]
    r = bench.policy_fidelity(q[0], k[0], v[0], keep[0], blocks, 128, 64, 1 / np.sqrt(128), window=3)
    # position-only: tile 0 plus tiles jmax-2 .. jmax of each block
    slots = []
    for b in blocks:
        jm = (min(b * 128 + 128, L) - 1) // 64
        tiles = {0} | set(range(max(0, jm - 2), jm + 1))
        for i in range(b * 128, min(b * 128 + 128, L)):
            slots.append(sum(1 for j in range(i + 1) if j // 64 in tiles))
    assert (r["position_only"]["slots"] == np.array(slots)).all()
    assert r["position_only"]["tiles"] == sum(len({0} | set(range(max(0, (min(b * 128 + 128, L) - 1) // 64 - 2),
                                                                     (min(b * 128 + 128, L) - 1) // 64 + 1)))
                                              for b in blocks)


def test_full_keep_is_exact(case):
    w, q, k, v, keep = case
    full = np.ones_like(keep[0])
    r = bench.policy_fidelity(q[0], k[0], v[0], full, [0, 5, 9], 128, 64, 1 / np.sqrt(128), window=100)
    for name in ("mala", "reference_mass", "position_only"):
        assert np.abs(r[name]["omitted"]).max() < 1e-12
        assert r[name]["rel"].max() < 1e-12
    rows = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in (0, 5, 9)])
    assert (r["mala"]["slots"] == rows + 1).all()


def test_position_window_is_closest():
    blocks, L = [0, 8, 16, 24], 4096
    for target in (10, 37, 80, 200):
        wsel, count = bench.position_window(blocks, 128, 64, L, 4, target)
        best = min(abs(count(x) - target) for x in range(1, 2 * 24 + 3))
        assert abs(count(wsel) - target) == best
