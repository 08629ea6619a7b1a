"""Pins of the CPU oracle against facts fixed independently of it.

Each test names the fact it checks.  Passages are cited from "MassAlloc
Attention: Let Attention Allocate Its Own Compute" (agihunt.info digest) by
paragraph topic.  Inputs are small seeded instances of the named workloads so
the whole file runs in well under a minute on CPU.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import dense
from synth import WORKLOADS, prefill_inputs, decode_inputs, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _prefill(name, L=None, heads=None, family="planted"):
    w = WORKLOADS[name]
    x = prefill_inputs(w, family=family, L=L, heads=heads)
    H = len(heads) if heads is not None else w.H
    hs = list(heads) if heads is not None else list(range(w.H))
    return w, [to_f64(x[n][:, hs], w.dtype) for n in ("q", "k", "v", "do")]


def _legal(L, bq, bk):
    nqb, nt = -(-L // bq), -(-L // bk)
    return np.array([[t * bk <= min(b * bq + bq, L) - 1 for t in range(nt)] for b in range(nqb)])


@pytest.fixture(scope="module")
def tiny():
    return _prefill("tiny")


@pytest.fixture(scope="module")
def small_bf16():
    # 8K-workload recipe, shortened to a ragged length (not a multiple of 128 or 64)
    return _prefill("mw8k", L=1000, heads=[0, 2, 5])


# ---------------------------------------------------------------- worked examples
@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "worked_examples.json")))["cases"],
                         ids=lambda c: c["name"])
def test_worked_example(case):
    """Hand-derived decisions (tests/golden/worked_examples.md); O and lse are the
    closed-form softmax over the hand-derived kept keys."""
    q = np.array(case["q"], float).reshape(1, 1, -1, 1)
    k = np.array(case["k"], float).reshape(1, 1, -1, 1)
    v = np.array(case["v"], float).reshape(1, 1, -1, 1)
    o, lse, keep, T = oracle.fwd(q, k, v, case["tau"], case["bq"], case["bk"], scale=case["scale"])
    exp_keep = np.array(case["keep"], np.uint8)
    assert (keep[0, 0] == exp_keep).all()
    for i, kk in enumerate(case["kept_keys"]):
        s = np.array([case["q"][i] * case["k"][j] for j in kk])
        z = sum(math.exp(x) for x in s)
        o_exp = sum(math.exp(x) * case["v"][j] for x, j in zip(s, kk)) / z
        assert abs(o[0, 0, i, 0] - o_exp) <= 1e-12 * abs(o_exp)
        assert abs(lse[0, 0, i] - math.log(z)) <= 1e-12


def test_worked_example_distant_row3_closed_form():
    """Row 3 of the first worked example, written out: O = (40e^2 + 10e^3)/(e^2 + e^3)."""
    q = np.ones((1, 1, 4, 1)); k = np.array([3.0, -3.0, 0.5, 2.0]).reshape(1, 1, 4, 1)
    v = np.array([10.0, 20.0, 30.0, 40.0]).reshape(1, 1, 4, 1)
    o, lse, keep, _ = oracle.fwd(q, k, v, 1.0, 1, 1, scale=1.0)
    e2, e3 = math.exp(2), math.exp(3)
    assert abs(o[0, 0, 3, 0] - (40 * e2 + 10 * e3) / (e2 + e3)) < 1e-12
    assert abs(lse[0, 0, 3] - math.log(e2 + e3)) < 1e-12


# ---------------------------------------------------------------- P1: tau = 0 is full attention
def test_tau0_fwd_equals_dense_tiny(tiny):
    """Savings paragraph: as tau -> 0 both passes recover full attention."""
    w, (q, k, v, do) = tiny
    o, lse, keep, _ = oracle.fwd(q, k, v, 0.0, w.bq, w.bk)
    od, ld = dense.fwd(q, k, v, 1 / math.sqrt(w.d))
    assert np.abs(o - od).max() <= 1e-12 * np.abs(od).max()
    assert np.abs(lse - ld).max() <= 1e-12 * np.abs(ld).max()
    assert keep[0, 0][_legal(w.L, w.bq, w.bk)].all()


def test_tau0_fwd_equals_dense_bf16_ragged(small_bf16):
    w, (q, k, v, do) = small_bf16
    o, lse, _, _ = oracle.fwd(q, k, v, 0.0, 128, 64)
    od, ld = dense.fwd(q, k, v, 1 / math.sqrt(w.d))
    assert np.abs(o - od).max() <= 1e-12 * np.abs(od).max()
    assert np.abs(lse - ld).max() <= 1e-12 * np.abs(ld).max()


# ---------------------------------------------------------------- P2: tau = 0 backward is the exact gradient
def test_dense_gradient_matches_finite_differences():
    """The dense analytic gradient (the tau=0 target) against central differences
    of the scalar loss sum(dO * O) on a 2-head, 64-token instance."""
    rng = np.random.default_rng(7)
    L, d = 64, 16
    scale = 1 / math.sqrt(d)
    for h in range(2):
        q, k, v, do = (rng.standard_normal((L, d)) for _ in range(4))
        dq, dk, dv = dense.bwd_head(q, k, v, do, scale)

        def loss(q_, k_, v_):
            return float((dense.fwd_head(q_, k_, v_, scale)[0] * do).sum())

        eps = 1e-6
        for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            for (i, c) in [(0, 0), (17, 3), (40, 9), (63, 15), (5, 1)]:
                a = [q.copy(), k.copy(), v.copy()]
                a[which][i, c] += eps
                lp = loss(*a)
                a[which][i, c] -= 2 * eps
                lm = loss(*a)
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - grad[i, c]) <= 1e-6 * max(1.0, abs(fd)), (which, i, c, fd, grad[i, c])


def test_tau0_bwd_equals_dense_gradient(tiny, small_bf16):
    for w, (q, k, v, do) in (tiny, small_bf16):
        bq, bk = (w.bq, w.bk) if w.dtype == "f32" else (128, 64)
        o, lse, _, _ = oracle.fwd(q, k, v, 0.0, bq, bk)
        dq, dk, dv, keep, _ = oracle.bwd(q, k, v, o, lse, do, 0.0, bq, bk)
        g = dense.bwd(q, k, v, do, 1 / math.sqrt(w.d))
        for a, b in zip((dq, dk, dv), g):
            assert np.abs(a - b).max() <= 1e-11 * np.abs(b).max()
        assert keep[0, 0][_legal(q.shape[2], bq, bk)].all()


# ---------------------------------------------------------------- P3: no empty row
@pytest.mark.parametrize("tau", [0.5, 1.0, 4.0, 64.0, math.inf])
def test_no_empty_row(small_bf16, tau):
    """Forward paragraph: the first legal tile is always kept, so no row is empty."""
    w, (q, k, v, do) = small_bf16
    o, lse, keep, T = oracle.fwd(q, k, v, tau, 128, 64)
    assert np.isfinite(lse).all() and np.isfinite(o).all()


# ---------------------------------------------------------------- P4: nesting
@pytest.mark.parametrize("tau", [0.5, 1.0, 2.0, 16.0])
def test_backward_support_nested_in_forward(small_bf16, tau):
    """MassAlloc Attention digest (agihunt.info), backward paragraph: the final
    normalizer sums every kept tile, so it is never smaller than the running one
    a forward test used; each backward ratio is at most its forward ratio and a
    tile forward skipped stays skipped in backward."""
    w, (q, k, v, do) = small_bf16
    o, lse, kf, _ = oracle.fwd(q, k, v, tau, 128, 64)
    _, _, _, kb, _ = oracle.bwd(q, k, v, o, lse, do, tau, 128, 64)
    assert (kb <= kf).all()
    if tau >= 2.0:
        assert kb.sum() < kf.sum()   # the inclusion is strict somewhere on these inputs


# ---------------------------------------------------------------- P5: omitted-mass bound
@pytest.mark.parametrize("tau", [0.25, 1.0, 8.0, 1000.0])
def test_omitted_mass_below_bound(tau):
    """Limits paragraph: per-row omitted mass stays below tau/(1+tau); checked by
    brute force against the dense softmax on inputs where many tiles skip."""
    w, (q, k, v, do) = _prefill("mw8k", L=700, heads=[2, 6, 9])
    o, lse, keep, _ = oracle.fwd(q, k, v, tau, 128, 64)
    worst = 0.0
    for h in range(q.shape[1]):
        P = dense.probs_head(q[0, h], k[0, h], 1 / math.sqrt(w.d))
        L = q.shape[2]
        mask = np.zeros((L, L), bool)
        for i in range(L):
            for t in range(-(-L // 64)):
                if keep[0, h, i // 128, t]:
                    mask[i, t * 64:(t + 1) * 64] = True
        om = (P * ~mask).sum(axis=1)
        assert (om < tau / (1 + tau)).all()
        worst = max(worst, om.max())
    if tau >= 8.0:
        assert worst > 1e-3   # the bound is exercised, not vacuous


# ---------------------------------------------------------------- P6: tau = +inf keeps only forced tiles
def test_tau_inf_forced_tiles_only(small_bf16):
    """Forward keeps exactly the tiles visited while some row is still empty (for
    128x64 tiles: the two diagonal-side tiles 2b+1 and 2b); the output is dense
    attention restricted to those keys.  Backward has no forced keep: all zero."""
    w, (q, k, v, do) = small_bf16
    L = q.shape[2]
    o, lse, keep, _ = oracle.fwd(q, k, v, math.inf, 128, 64)
    nqb, nt = keep.shape[2:]
    exp = np.zeros((nqb, nt), np.uint8)
    for b in range(nqb):
        jmax = (min(b * 128 + 128, L) - 1) // 64
        exp[b, jmax] = 1
        if b * 128 < jmax * 64:   # rows b*128 .. see nothing in the last tile
            exp[b, jmax - 1] = 1
    for h in range(q.shape[1]):
        assert (keep[0, h] == exp).all()
        mask = np.zeros((L, L), bool)
        for i in range(L):
            for t in range(nt):
                if exp[i // 128, t]:
                    mask[i, t * 64:(t + 1) * 64] = True
        od, ld = dense.fwd_head(q[0, h], k[0, h], v[0, h], 1 / math.sqrt(w.d), key_mask=mask)
        assert np.abs(o[0, h] - od).max() <= 1e-12 * np.abs(od).max()
        assert np.abs(lse[0, h] - ld).max() <= 1e-12
    dq, dk, dv, kb, _ = oracle.bwd(q, k, v, o, lse, do, math.inf, 128, 64)
    assert kb.sum() == 0
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()


# ---------------------------------------------------------------- P10: kept-set restricted dense
@pytest.mark.parametrize("tau", [1.0, 4.0])
def test_fwd_output_is_dense_over_kept_keys(small_bf16, tau):
    """The online update is exact on the kept set: O_i and lse_i equal softmax
    attention of row i over the keys of its block's kept tiles."""
    w, (q, k, v, do) = small_bf16
    L = q.shape[2]
    o, lse, keep, _ = oracle.fwd(q, k, v, tau, 128, 64)
    for h in range(q.shape[1]):
        mask = np.zeros((L, L), bool)
        for i in range(L):
            for t in range(keep.shape[3]):
                if keep[0, h, i // 128, t]:
                    mask[i, t * 64:(t + 1) * 64] = True
        od, ld = dense.fwd_head(q[0, h], k[0, h], v[0, h], 1 / math.sqrt(w.d), key_mask=mask)
        assert np.abs(o[0, h] - od).max() <= 1e-12 * np.abs(od).max()
        assert np.abs(lse[0, h] - ld).max() <= 1e-12


# ---------------------------------------------------------------- P7: decision brute force
@pytest.mark.parametrize("tau", [1.0, 4.0, 16.0])
def test_decisions_by_direct_sums(tau):
    """Every tile's statistic recomputed without online rescaling: for each row the
    running normalizer is the plain sum of exp(s) over keys of previously kept
    tiles, T = max over voting rows of max_j exp(s_ij)/Z_i * Lq_i/tau."""
    w, (q, k, v, do) = _prefill("mw8k", L=520, heads=[2, 5])
    bq, bk = 128, 64
    o, lse, keep, T = oracle.fwd(q, k, v, tau, bq, bk)
    L = q.shape[2]
    scale = 1 / math.sqrt(w.d)
    flips = 0
    for h in range(q.shape[1]):
        S = scale * q[0, h] @ k[0, h].T
        for b in range(keep.shape[2]):
            rows = range(b * bq, min(b * bq + bq, L))
            Z = {i: 0.0 for i in rows}
            jmax = (max(rows)) // bk
            for t in range(jmax, -1, -1):
                cols = range(t * bk, min(t * bk + bk, L))
                Tt = 0.0
                for i in rows:
                    vis = [j for j in cols if j <= i]
                    if not vis:
                        continue
                    if Z[i] == 0.0:
                        Tt = math.inf
                        continue
                    r = max(math.exp(S[i, j]) for j in vis) / Z[i]
                    Tt = max(Tt, r * (i + 1) / tau)
                kp = Tt >= 1.0
                assert kp == bool(keep[0, h, b, t]), (h, b, t, Tt)
                if math.isfinite(Tt):
                    assert abs(Tt - T[0, h, b, t]) <= 1e-9 * Tt
                if kp:
                    for i in rows:
                        Z[i] += sum(math.exp(S[i, j]) for j in cols if j <= i)
                flips += not kp
    assert flips > 0


@pytest.mark.parametrize("tau", [0.5, 1.0, 4.0])
def test_backward_statistic_by_direct_probabilities(tau):
    """Backward paragraph: every legal tile is tested against the final
    log-normalizer.  Recomputed here from P_ij = exp(s_ij - lse_i) with the
    lse the forward wrote: T = max over rows with a visible key of
    max_j P_ij * Lq_i / tau, kept iff T >= 1, with no forced keep; the
    oracle's backward T and decisions must match."""
    w, (q, k, v, do) = _prefill("mw8k", L=520, heads=[1, 4])
    bq, bk = 128, 64
    o, lse, _, _ = oracle.fwd(q, k, v, tau, bq, bk)
    _, _, _, kb, Tb = oracle.bwd(q, k, v, o, lse, do, tau, bq, bk)
    L = q.shape[2]
    scale = 1 / math.sqrt(w.d)
    skipped = 0
    for h in range(q.shape[1]):
        P = np.exp(scale * q[0, h] @ k[0, h].T - lse[0, h][:, None])
        for b in range(kb.shape[2]):
            rows = np.arange(b * bq, min(b * bq + bq, L))
            for t in range(rows[-1] // bk + 1):
                cols = np.arange(t * bk, min(t * bk + bk, L))
                vis = cols[None, :] <= rows[:, None]
                voting = vis.any(axis=1)
                ratio = np.where(vis, P[np.ix_(rows, cols)], 0.0).max(axis=1) * (rows + 1) / tau
                Tt = ratio[voting].max()
                assert abs(Tt - Tb[0, h, b, t]) <= 1e-9 * Tt, (h, b, t)
                assert bool(kb[0, h, b, t]) == (Tt >= 1.0), (h, b, t, Tt)
                skipped += Tt < 1.0
    assert skipped > 0


# ---------------------------------------------------------------- P9: log-domain form of the test
@pytest.mark.parametrize("tau", [0.5, 1.0, 4.0])
def test_log_domain_test_gives_same_decisions(tau):
    """The GPU kernels test rowmax_i >= m_i + ln(l_i) + ln(tau) - ln(Lq_i) instead
    of the ratio form.  Both forms, run side by side in fp64 on the same running
    state, agree on every tile of these inputs (they differ only on exact ties)."""
    w, (q, k, v, do) = _prefill("mw8k", L=384, heads=[2])
    bq, bk = 128, 64
    _, _, keep, _ = oracle.fwd(q, k, v, tau, bq, bk)
    S = q[0, 0] @ k[0, 0].T / math.sqrt(w.d)
    L = S.shape[0]
    for b in range(keep.shape[2]):
        rows = list(range(b * bq, min(b * bq + bq, L)))
        m = {i: -math.inf for i in rows}
        lsum = {i: 0.0 for i in rows}
        for t in range((rows[-1]) // bk, -1, -1):
            kp_log = False
            for i in rows:
                vis = [j for j in range(t * bk, min(t * bk + bk, L)) if j <= i]
                if not vis:
                    continue
                if lsum[i] == 0.0:
                    kp_log = True
                    continue
                thr = m[i] + math.log(lsum[i]) + math.log(tau) - math.log(i + 1)
                kp_log |= max(S[i, j] for j in vis) >= thr
            assert kp_log == bool(keep[0, 0, b, t])
            if kp_log:
                for i in rows:
                    vis = [j for j in range(t * bk, min(t * bk + bk, L)) if j <= i]
                    if not vis:
                        continue
                    mn = max(m[i], max(S[i, j] for j in vis))
                    lsum[i] = lsum[i] * math.exp(m[i] - mn) + sum(math.exp(S[i, j] - mn) for j in vis)
                    m[i] = mn


# ---------------------------------------------------------------- replay mode
def test_replay_band_only_overrides_near_threshold(small_bf16):
    """Replay adopts foreign decisions only where |T - 1| <= band: flipping every
    decision outside the band changes nothing."""
    w, (q, k, v, do) = small_bf16
    o, lse, keep, T = oracle.fwd(q, k, v, 1.0, 128, 64)
    o2, lse2, keep2, T2 = oracle.fwd(q, k, v, 1.0, 128, 64, replay=1 - keep, band=1e-4)
    near = np.isfinite(T) & (np.abs(T - 1) <= 1e-4)
    assert (keep2[~near] == keep[~near]).all()
    o3, _, keep3, T3 = oracle.fwd(q, k, v, 1.0, 128, 64, replay=1 - keep, band=np.inf)
    finite = np.isfinite(T3)
    assert (keep3[finite] != keep[finite]).any()


# ---------------------------------------------------------------- P8: decode
def _decode_small(Lk=1000):
    w = WORKLOADS["decode128k"]
    x = decode_inputs(w, Lk=Lk, batches=[0])
    return w, to_f64(x["q"][:1], w.dtype), to_f64(x["k"][:1], w.dtype), to_f64(x["v"][:1], w.dtype)


def test_decode_tau0_is_dense_single_query():
    w, q, kc, vc = _decode_small(1000)
    o, lse, keep, _ = oracle.decode(q, kc, vc, 1000, 0.0, 256, 64)
    G = w.group
    for h in range(w.H):
        g = h // G
        s = kc[0, g] @ q[0, h] / math.sqrt(w.d)
        p = np.exp(s - s.max())
        assert np.abs(o[0, h] - p @ vc[0, g] / p.sum()).max() <= 1e-12 * np.abs(o[0, h]).max()
        assert abs(lse[0, h] - (s.max() + math.log(p.sum()))) <= 1e-12


def test_decode_split_independence_at_tau0():
    w, q, kc, vc = _decode_small(1000)
    o1, l1, _, _ = oracle.decode(q, kc, vc, 1000, 0.0, 128, 64)
    o2, l2, _, _ = oracle.decode(q, kc, vc, 1000, 0.0, 4096, 64)
    assert np.abs(o1 - o2).max() <= 1e-12 * np.abs(o2).max()
    assert np.abs(l1 - l2).max() <= 1e-12


@pytest.mark.parametrize("tau", [1.0, 8.0])
def test_decode_one_split_one_row_equals_forward_row(tau):
    """With a single partition and a one-row vote, decode of the query at
    position Lk-1 is the forward pass of that row with a one-row block."""
    w, q, kc, vc = _decode_small(777)
    Lk = 777
    o, lse, keep, T = oracle.decode(q, kc, vc, Lk, tau, 4096, 64, rows_per_vote=1)
    for h in (0, 5, 30):
        g = h // w.group
        qq = np.zeros((1, 1, Lk, w.d))
        qq[0, 0, Lk - 1] = q[0, h]
        kk = kc[0, g, :Lk][None, None]
        vv = vc[0, g, :Lk][None, None]
        of, lf, kf, Tf = oracle.fwd(qq, kk, vv, tau, 1, 64, qblocks=[Lk - 1])
        assert np.abs(o[0, h] - of[0, 0, Lk - 1]).max() <= 1e-12 * np.abs(of[0, 0, Lk - 1]).max()
        assert abs(lse[0, h] - lf[0, 0, Lk - 1]) <= 1e-12
        nt = -(-Lk // 64)
        assert (keep[0, g, h % w.group, 0, :nt] == kf[0, 0, Lk - 1, :nt]).all()


@pytest.mark.parametrize("tau,rpv", [(1.0, None), (4.0, None), (4.0, 2), (16.0, 1)])
def test_decode_decisions_by_direct_sums(tau, rpv):
    """Decode's statistic recomputed without online rescaling: in each
    partition, tiles are visited newest first, each row's normalizer is the
    plain sum of exp(s) over keys of previously kept tiles of that partition
    (none at the first tile, which is therefore kept), and a vote group's
    T = max over its rows of max_j exp(s_j)/Z * Lk/tau."""
    w, q, kc, vc = _decode_small(1500)
    Lk, S, bk = 1500, 512, 64
    o, lse, keep, T = oracle.decode(q, kc, vc, Lk, tau, S, bk, rows_per_vote=rpv)
    G = w.group
    R = G if rpv is None else rpv
    nsplit, tps = oracle.decode_shapes(Lk, S, bk)
    skipped = 0
    for g in range(kc.shape[1]):
        s = q[0, g * G:(g + 1) * G] @ kc[0, g, :Lk].T / math.sqrt(w.d)
        for vg in range(G // R):
            rows = range(vg * R, vg * R + R)
            for p in range(nsplit):
                Z = {r: 0.0 for r in rows}
                k1 = min(p * S + S, Lk)
                for t in range(-(-(k1 - p * S) // bk) - 1, -1, -1):
                    cols = range(p * S + t * bk, min(p * S + t * bk + bk, k1))
                    Tt = 0.0
                    for r in rows:
                        if Z[r] == 0.0:
                            Tt = math.inf
                            continue
                        Tt = max(Tt, max(math.exp(s[r, j]) for j in cols) / Z[r] * Lk / tau)
                    kp = Tt >= 1.0
                    assert kp == bool(keep[0, g, vg, p, t]), (g, vg, p, t, Tt)
                    if math.isfinite(Tt):
                        assert abs(Tt - T[0, g, vg, p, t]) <= 1e-9 * Tt, (g, vg, p, t)
                    if kp:
                        for r in rows:
                            Z[r] += sum(math.exp(s[r, j]) for j in cols)
                    skipped += not kp
    assert skipped > 0


@pytest.mark.parametrize("tau", [1.0, 16.0])
def test_decode_is_dense_over_kept_keys_and_bounded(tau):
    """The exact merge of partition states makes decode output the softmax over
    the union of kept tiles; per partition the omitted mass obeys the bound."""
    w, q, kc, vc = _decode_small(1500)
    Lk, S, bk = 1500, 512, 64
    o, lse, keep, T = oracle.decode(q, kc, vc, Lk, tau, S, bk)
    G = w.group
    nsplit, tps = oracle.decode_shapes(Lk, S, bk)
    skipped_any = False
    for h in range(w.H):
        g = h // G
        s = kc[0, g, :Lk] @ q[0, h] / math.sqrt(w.d)
        mask = np.zeros(Lk, bool)
        for p in range(nsplit):
            for t in range(tps):
                if keep[0, g, 0, p, t]:
                    mask[p * S + t * bk: min(p * S + (t + 1) * bk, (p + 1) * S, Lk)] = True
        skipped_any |= not mask.all()
        e = np.exp(s[mask] - s[mask].max())
        assert np.abs(o[0, h] - e @ vc[0, g, :Lk][mask] / e.sum()).max() <= 1e-12 * np.abs(o[0, h]).max()
        P = np.exp(s - s.max()); P /= P.sum()
        assert P[~mask].sum() < tau / (1 + tau)
        # each partition's first visited tile is kept
        for p in range(nsplit):
            nt = -(-(min((p + 1) * S, Lk) - p * S) // bk)
            assert keep[0, g, 0, p, nt - 1] == 1
    if tau >= 16.0:
        assert skipped_any


def test_invalid_tau_rejected():
    q = np.zeros((1, 1, 4, 2))
    for bad in (-1.0, float("nan")):
        with pytest.raises(RuntimeError):
            oracle.fwd(q, q, q, bad, 2, 2)


# ---------------------------------------------------------------- grouped K/V heads (GQA)
def _gqa_small(L=700):
    w = WORKLOADS["gqa8k"]
    x = prefill_inputs(w, L=L, heads=range(4))  # query heads 0..3 = K/V head 0 (one group)
    q = to_f64(x["q"][:, :4], w.dtype)
    k, v = (to_f64(x[n][:, :1], w.dtype) for n in ("k", "v"))
    do = to_f64(x["do"][:, :4], w.dtype)
    return w, q, k, v, do


def test_gqa_tau0_equals_dense_with_shared_kv():
    """Grouped-query attention: every query head of a group attends with the
    group's one K/V head, so at tau=0 the forward is dense attention with that
    K/V repeated per head, and the gradient of the shared K (V) is the sum of
    the per-head gradients (a tensor used by several heads)."""
    w, q, k, v, do = _gqa_small()
    G = q.shape[1]
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    scale = 1 / math.sqrt(w.d)
    o, lse, _, _ = oracle.fwd(q, k, v, 0.0, w.bq, w.bk)
    od, ld = dense.fwd(q, kr, vr, scale)
    assert np.abs(o - od).max() <= 1e-12 * np.abs(od).max()
    assert np.abs(lse - ld).max() <= 1e-12 * np.abs(ld).max()
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, o, lse, do, 0.0, w.bq, w.bk)
    gq, gk, gv = dense.bwd(q, kr, vr, do, scale)
    assert dk.shape == k.shape and dv.shape == v.shape
    assert np.abs(dq - gq).max() <= 1e-11 * np.abs(gq).max()
    assert np.abs(dk - gk.sum(axis=1, keepdims=True)).max() <= 1e-11 * np.abs(gk).max()
    assert np.abs(dv - gv.sum(axis=1, keepdims=True)).max() <= 1e-11 * np.abs(gv).max()


@pytest.mark.parametrize("tau", [1.0, 4.0])
def test_gqa_gated_equals_per_head_runs(tau):
    """Decisions are per query head (each head's rows vote on its own tiles),
    so with grouped K/V the gated result equals running every query head on
    its own copy of the shared K/V, with the K/V gradients summed."""
    w, q, k, v, do = _gqa_small()
    G = q.shape[1]
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o, lse, keep, _ = oracle.fwd(q, k, v, tau, w.bq, w.bk)
    o2, lse2, keep2, _ = oracle.fwd(q, kr, vr, tau, w.bq, w.bk)
    assert (keep == keep2).all() and (keep == 0).any()
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    dq, dk, dv, kb, _ = oracle.bwd(q, k, v, o, lse, do, tau, w.bq, w.bk)
    dq2, dk2, dv2, kb2, _ = oracle.bwd(q, kr, vr, o, lse, do, tau, w.bq, w.bk)
    assert (kb == kb2).all()
    assert np.array_equal(dq, dq2)
    assert np.abs(dk - dk2.sum(axis=1, keepdims=True)).max() <= 1e-12 * np.abs(dk).max()
    assert np.abs(dv - dv2.sum(axis=1, keepdims=True)).max() <= 1e-12 * np.abs(dv).max()


# ---------------------------------------------------------------- chunked prefill (query offset)
def _chunk_case(P, Lq=300, heads=(2, 6)):
    """A whole planted sequence of length P + Lq; the chunk is its last Lq rows."""
    w, (q, k, v, do) = _prefill("mw8k", L=P + Lq, heads=list(heads))
    return w, q, k, v


@pytest.mark.parametrize("P", [0, 256, 333])
def test_chunk_tau0_equals_dense_rows(P):
    """Threshold paragraph: Lq is a row's count of visible keys, so a chunk at
    offset P is causal attention of rows P.. over keys 0..P+i.  At tau=0 the
    chunked forward equals those rows of dense causal attention."""
    w, q, k, v = _chunk_case(P)
    o, lse, keep, _ = oracle.fwd_chunk(q[:, :, P:], k, v, P, 0.0, 128, 64)
    od, ld = dense.fwd(q, k, v, 1 / math.sqrt(w.d))
    assert np.abs(o - od[:, :, P:]).max() <= 1e-12 * np.abs(od).max()
    assert np.abs(lse - ld[:, :, P:]).max() <= 1e-12 * np.abs(ld).max()


@pytest.mark.parametrize("tau", [1.0, 4.0])
def test_chunk_aligned_equals_whole_sequence_blocks(tau):
    """A query block's decisions and outputs depend only on its own rows and
    the keys they see, so a chunk that starts on a query-block boundary
    reproduces the whole-sequence forward's blocks exactly."""
    P = 256
    w, q, k, v = _chunk_case(P)
    o, lse, keep, _ = oracle.fwd_chunk(q[:, :, P:], k, v, P, tau, 128, 64)
    of, lf, kf, _ = oracle.fwd(q, k, v, tau, 128, 64)
    assert (keep == kf[:, :, P // 128:]).all() and (keep == 0).any()
    assert np.array_equal(o, of[:, :, P:]) and np.array_equal(lse, lf[:, :, P:])


@pytest.mark.parametrize("tau", [1.0, 8.0])
def test_chunk_unaligned_dense_over_kept_and_bounded(tau):
    """Unaligned offset: the output is softmax attention over the keys of the
    kept tiles (exact online update), the first tile visited is kept, and
    every row's omitted mass stays below tau/(1+tau) (limits paragraph)."""
    P = 333
    w, q, k, v = _chunk_case(P)
    Lq, Lk = q.shape[2] - P, q.shape[2]
    o, lse, keep, _ = oracle.fwd_chunk(q[:, :, P:], k, v, P, tau, 128, 64)
    scale = 1 / math.sqrt(w.d)
    for h in range(q.shape[1]):
        Pd = dense.probs_head(q[0, h], k[0, h], scale)[P:]
        mask = np.zeros((Lq, Lk), bool)
        for i in range(Lq):
            jmax = (P + (i // 128) * 128 + min(128, Lq - (i // 128) * 128) - 1) // 64
            assert keep[0, h, i // 128, jmax]
            for t in range(keep.shape[3]):
                if keep[0, h, i // 128, t]:
                    mask[i, t * 64:(t + 1) * 64] = True
        full = np.ones((Lk, Lk), bool)  # rows before the chunk: unused here
        full[P:] = mask
        od, ld = dense.fwd_head(q[0, h], k[0, h], v[0, h], scale, key_mask=full)
        assert np.abs(o[0, h] - od[P:]).max() <= 1e-12 * np.abs(od[P:]).max()
        om = (Pd * ~mask).sum(axis=1)
        assert (om < tau / (1 + tau)).all()


# ---------------------------------------------------------------- seeded decode partitions
def _seeded_tiles_mask(keep_g, Lk, S, bk):
    """Key mask of the kept tiles of one vote group of the seeded decode."""
    nsplit, tps = oracle.seeded_decode_shapes(Lk, S, bk)
    jd = (Lk - 1) // bk
    mask = np.zeros(Lk, bool)
    for p in range(nsplit):
        hi = jd - p * tps
        lo = max(0, hi - tps + 1)
        for t in range(hi - lo + 1):
            if keep_g[p, t]:
                mask[(lo + t) * bk: min((lo + t + 1) * bk, Lk)] = True
    return mask


@pytest.mark.parametrize("tau", [1.0, 8.0])
def test_seeded_decode_one_partition_is_plain_decode(tau):
    """With one partition there is nothing to seed: the seeded decode is the
    plain decode (same tiles from key 0, same visit order, empty start)."""
    w, q, kc, vc = _decode_small(777)
    o1, l1, k1, _ = oracle.decode(q, kc, vc, 777, tau, 1024, 64)
    o2, l2, k2, _ = oracle.decode_seeded(q, kc, vc, 777, tau, 1024, 64)
    assert (k1 == k2).all()
    assert np.abs(o1 - o2).max() <= 1e-12 * np.abs(o1).max()
    assert np.abs(l1 - l2).max() <= 1e-12


def test_seeded_decode_tau0_is_dense():
    w, q, kc, vc = _decode_small(1000)
    o, lse, keep, _ = oracle.decode_seeded(q, kc, vc, 1000, 0.0, 256, 64)
    for h in range(w.H):
        g = h // w.group
        s = kc[0, g, :1000] @ q[0, h] / math.sqrt(w.d)
        p = np.exp(s - s.max())
        assert np.abs(o[0, h] - p @ vc[0, g, :1000] / p.sum()).max() <= 1e-12 * np.abs(o[0, h]).max()
        assert abs(lse[0, h] - (s.max() + math.log(p.sum()))) <= 1e-12


def test_seeded_partition0_is_plain_last_partition():
    """When Lk is a multiple of the partition size the newest partition of the
    seeded decode is the last partition of the plain decode (same tiles, both
    start empty), so its decisions and state are the same."""
    w, q, kc, vc = _decode_small(1536)
    Lk, S, bk = 1536, 512, 64
    G = w.group
    for g in (0, 3):
        r1 = oracle.decode_group_partials(q[0, g * G:(g + 1) * G], kc[0, g], vc[0, g], Lk, 4.0, S, bk)
        r2 = oracle.decode_seeded_group_partials(q[0, g * G:(g + 1) * G], kc[0, g], vc[0, g], Lk, 4.0, S, bk)
        assert (r1[2][:, 2] == r2[2][:, 0]).all()
        for a, b in zip(r1[4:], r2[4:]):
            assert np.array_equal(a[:, 2], b[:, 0])


def test_seeded_decode_keeps_nothing_by_force():
    """Constructed case: one dominant key at the newest position, every other
    key orthogonal to the queries (score 0).  Partition 0 keeps its diagonal
    tile (forced, empty state) and skips the rest (ratio e^-30 < tau/Lk); every
    older partition is tested against that normalizer and skips everything,
    so the output is softmax attention over the diagonal tile.  The plain
    decode starts each noise-only partition empty: its first visited tile is
    forced, and the rest then pass (ratio 1/(64 n) >= tau/Lk), so it keeps
    every tile of the three older partitions."""
    Lk, S, bk, d, G = 1000, 256, 64, 128, 4
    rng = np.random.default_rng(7)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = np.tile(u * math.sqrt(30.0 * math.sqrt(d)), (1, G, 1))  # score with k = u * sqrt(30 sqrt(d)) is 30
    k = np.zeros((1, 1, Lk, d))
    k[0, 0, Lk - 1] = u * math.sqrt(30.0 * math.sqrt(d))
    v = rng.standard_normal((1, 1, Lk, d))
    o, lse, keep, T = oracle.decode_seeded(q, k, v, Lk, 1.0, S, bk)
    nsplit, tps = oracle.seeded_decode_shapes(Lk, S, bk)
    assert nsplit == 4
    assert keep.sum() == 1 and keep[0, 0, 0, 0, tps - 1] == 1  # only the diagonal tile (tile 15)
    jd = (Lk - 1) // bk
    s = np.zeros(Lk - jd * bk)
    s[-1] = 30.0
    p = np.exp(s - s.max())
    ref = p @ v[0, 0, jd * bk:Lk] / p.sum()
    for r in range(G):
        assert np.abs(o[0, r] - ref).max() <= 1e-12 * np.abs(ref).max()
        assert abs(lse[0, r] - (30.0 + math.log(p.sum()))) <= 1e-12
    _, _, keep_plain, _ = oracle.decode(q, k, v, Lk, 1.0, S, bk)
    assert keep_plain[0, 0, 0, :3].all() and keep_plain[0, 0, 0, 3].sum() == 1


@pytest.mark.parametrize("tau,rpv", [(1.0, None), (4.0, 2), (16.0, 1)])
def test_seeded_decode_decisions_by_direct_sums(tau, rpv):
    """Seeded decode recomputed with plain sums: partition 0 is the newest
    split_keys/bk tiles and starts with an empty normalizer; each older
    partition (tiles counted back from there, the oldest one ragged) starts
    from partition 0's final sum and adds its own kept tiles, newest first;
    a vote group's T = max over its rows of max_j exp(s_j)/Z * Lk/tau."""
    w, q, kc, vc = _decode_small(1500)
    Lk, S, bk = 1500, 256, 64
    o, lse, keep, T = oracle.decode_seeded(q, kc, vc, Lk, tau, S, bk, rows_per_vote=rpv)
    G = w.group
    R = G if rpv is None else rpv
    tps, jd = S // bk, (Lk - 1) // bk
    nsplit = -(-(jd + 1) // tps)
    assert keep.shape[3] == nsplit
    skipped = 0
    for g in range(kc.shape[1]):
        s = q[0, g * G:(g + 1) * G] @ kc[0, g, :Lk].T / math.sqrt(w.d)
        for vg in range(G // R):
            rows = range(vg * R, vg * R + R)
            Z0 = None
            for p in range(nsplit):
                Z = {r: 0.0 for r in rows} if p == 0 else dict(Z0)
                hi = jd - p * tps
                lo = max(hi - tps + 1, 0)
                for j in range(hi, lo - 1, -1):
                    cols = range(j * bk, min(j * bk + bk, Lk))
                    Tt = 0.0
                    for r in rows:
                        if Z[r] == 0.0:
                            Tt = math.inf
                            continue
                        Tt = max(Tt, max(math.exp(s[r, c]) for c in cols) / Z[r] * Lk / tau)
                    kp = Tt >= 1.0
                    assert kp == bool(keep[0, g, vg, p, j - lo]), (g, vg, p, j, Tt)
                    if math.isfinite(Tt):
                        assert abs(Tt - T[0, g, vg, p, j - lo]) <= 1e-9 * Tt, (g, vg, p, j)
                    if kp:
                        for r in rows:
                            Z[r] += sum(math.exp(s[r, c]) for c in cols)
                    skipped += not kp
                if p == 0:
                    Z0 = Z
    assert skipped > 0


@pytest.mark.parametrize("tau", [1.0, 16.0])
def test_seeded_decode_is_dense_over_kept_keys_and_bounded(tau):
    """The output is softmax attention over the union of kept tiles, and the
    omitted mass obeys the tau/(1+tau) bound: every skipped key's weight is
    below tau/Lk of a normalizer made of kept keys only."""
    w, q, kc, vc = _decode_small(1500)
    Lk, S, bk = 1500, 512, 64
    o, lse, keep, T = oracle.decode_seeded(q, kc, vc, Lk, tau, S, bk)
    skipped = 0
    for h in range(w.H):
        g = h // w.group
        mask = _seeded_tiles_mask(keep[0, g, 0], Lk, S, bk)
        skipped += int((~mask).sum())
        s = kc[0, g, :Lk] @ q[0, h] / math.sqrt(w.d)
        e = np.exp(s[mask] - s[mask].max())
        assert np.abs(o[0, h] - e @ vc[0, g, :Lk][mask] / e.sum()).max() <= 1e-12 * np.abs(o[0, h]).max()
        P = np.exp(s - s.max())
        P /= P.sum()
        assert P[~mask].sum() < tau / (1 + tau)
        assert keep[0, g, 0, 0, oracle.seeded_decode_shapes(Lk, S, bk)[1] - 1] == 1  # diagonal tile
    assert skipped > 0


def test_chunk_sampled_blocks_equal_full():
    """Computing only some query blocks of a chunk gives exactly those blocks
    of the full computation (every block's decisions depend on its own rows
    only); the others are left unset."""
    w = WORKLOADS["gqa8k"]
    P, Lq = 300, 400
    x = prefill_inputs(w, L=P + Lq, heads=range(4))
    q = to_f64(np.ascontiguousarray(x["q"][:, :4, P:]), w.dtype)
    k, v = (to_f64(x[n][:, :1], w.dtype) for n in ("k", "v"))
    o, lse, keep, T = oracle.fwd_chunk(q, k, v, P, 1.0, 128, 64)
    o2, lse2, keep2, T2 = oracle.fwd_chunk(q, k, v, P, 1.0, 128, 64, qblocks=[1, 3])
    rows = np.r_[128:256, 384:400]
    assert np.array_equal(o2[:, :, rows], o[:, :, rows]) and np.array_equal(lse2[:, :, rows], lse[:, :, rows])
    assert np.array_equal(keep2[:, :, [1, 3]], keep[:, :, [1, 3]])
    assert np.isnan(o2[:, :, :128]).all() and (keep2[:, :, [0, 2]] == 0).all()


# ---------------------------------------------------------------- row 0 of the backward
@pytest.mark.parametrize("tau", [0.5, 1.0, 2.0])
def test_backward_row0_probability_is_one(tau):
    """Forward paragraph: the first tile a block visits is always kept, and row
    0 sees only key 0, so its final normalizer is exp(s_00) and P_00 = 1.  With
    a single row the backward statistic is then exactly 1/tau (kept iff
    tau <= 1; equality keeps), and a kept tile gives dV_0 = dO_0 and
    dK_0 = dQ_0 = 0 (dS_00 = dP_00 - D_0 = <dO_0, v_0 - O_0> with O_0 = v_0)."""
    w, (q, k, v, do) = _prefill("mw8k", L=1, heads=[0, 3])
    o, lse, _, _ = oracle.fwd(q, k, v, tau, 128, 64)
    assert np.array_equal(o, v)
    # an lse off by a rounding error does not move row 0's decision
    lse_r = lse * (1 + 3e-8)
    dq, dk, dv, kb, Tb = oracle.bwd(q, k, v, o, lse_r, do, tau, 128, 64)
    assert (Tb[..., 0, 0] == 1.0 / tau).all()
    assert (kb[..., 0, 0] == (1 if tau <= 1.0 else 0)).all()
    if tau <= 1.0:
        assert np.array_equal(dv, do) and not dk.any() and not dq.any()
    else:
        assert not dv.any() and not dk.any() and not dq.any()


# ---------------------------------------------------------------- error scales of the rows
def _kept_keys(keep, i, bq, bk):
    """Keys of row i inside the tiles its block kept."""
    b = i // bq
    return [j for j in range(i + 1) if keep[b, j // bk]]


@pytest.mark.parametrize("tau", [1.0, 4.0])
def test_forward_row_error_scale(tau):
    """rs_i = sqrt(sum_j (p_ij |v_j|)^2) over the row's kept keys: for a row with
    one key it is |O_i| (row 0: O_0 = v_0); by Cauchy-Schwarz
    |O_i| <= sqrt(n_i) rs_i for a row with n_i kept keys; and it never exceeds
    max_j |v_j| (the p_ij sum to 1)."""
    w, (q, k, v, do) = _prefill("mw8k", L=600, heads=[1, 6])
    o, lse, keep, T, rs = oracle.fwd(q, k, v, tau, 128, 64, scales=True)
    vmax = np.linalg.norm(v, axis=-1).max()
    for h in range(2):
        on = np.linalg.norm(o[0, h], axis=-1)
        assert abs(rs[0, h, 0] - on[0]) <= 1e-12 * on[0]
        assert abs(rs[0, h, 0] - np.linalg.norm(v[0, h, 0])) <= 1e-12 * on[0]
        for i in range(q.shape[2]):
            n = len(_kept_keys(keep[0, h], i, 128, 64))
            assert on[i] <= math.sqrt(n) * rs[0, h, i] * (1 + 1e-12)
            assert rs[0, h, i] <= vmax * (1 + 1e-12)


@pytest.mark.parametrize("tau", [1.0, 4.0])
def test_backward_row_error_scales(tau):
    """The backward error scales (oracle_bwd_head): the last key is seen by the
    last row only, so its dK and dV rows are single terms and equal their
    scales rk, rv; every row obeys Cauchy-Schwarz, |X_i| <= sqrt(n_i) r_i with
    n_i terms; and |dS_ij| = P_ij |dP_ij - D_i| <= P_ij (a_ij + b_i), so each
    r is at most its c."""
    w, (q, k, v, do) = _prefill("mw8k", L=600, heads=[1, 6])
    o, lse, _, _ = oracle.fwd(q, k, v, tau, 128, 64)
    dq, dk, dv, kb, Tb, sc = oracle.bwd(q, k, v, o, lse, do, tau, 128, 64, scales=True)
    L = q.shape[2]
    for h in range(2):
        nk, nv = np.linalg.norm(dk[0, h], axis=-1), np.linalg.norm(dv[0, h], axis=-1)
        nq = np.linalg.norm(dq[0, h], axis=-1)
        if kb[0, h, (L - 1) // 128, (L - 1) // 64]:
            assert abs(sc["rk"][0, h, L - 1] - nk[L - 1]) <= 1e-9 * max(nk[L - 1], 1e-300)
            assert abs(sc["rv"][0, h, L - 1] - nv[L - 1]) <= 1e-12 * nv[L - 1]
        for i in range(L):
            nqi = len(_kept_keys(kb[0, h], i, 128, 64))
            assert nq[i] <= math.sqrt(max(nqi, 1)) * sc["rq"][0, h, i] * (1 + 1e-9) + 1e-300
            rows_j = [r for r in range(i, L) if kb[0, h, r // 128, i // 64]]
            assert nk[i] <= math.sqrt(max(len(rows_j), 1)) * sc["rk"][0, h, i] * (1 + 1e-9) + 1e-300
            assert nv[i] <= math.sqrt(max(len(rows_j), 1)) * sc["rv"][0, h, i] * (1 + 1e-9) + 1e-300
        assert (sc["rq"][0, h] <= sc["cq"][0, h] * (1 + 1e-12)).all()
        assert (sc["rk"][0, h] <= sc["ck"][0, h] * (1 + 1e-12)).all()
        assert (sc["rv"][0, h] > 0).any() and (sc["rq"][0, h] > 0).any()
