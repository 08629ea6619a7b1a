"""GPU parity at the full workload sizes, on sampled outputs.

The GPU runs the whole workload exactly as the bench launches it; the oracle
recomputes sampled query blocks (forward decisions, O, lse, dQ), sampled key
tiles (dK, dV) and sampled decode groups one by one -- every MALA decision of a
query block depends on that block's rows only, so a sampled block is checked
exactly, not approximately.  Same rules as the small-size parity tests
(tests/parity.py): forward and decode decisions outside the |T-1| <= 1e-4 band
identical (band tiles printed), backward decisions and kept counts identical
to the free-running oracle, O and gradients within their tensor and per-row
bounds; the backward support is nested in the forward's on every legal tile.
"""
import functools

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, decode_inputs, prefill_inputs, to_f64
from tests.parity import (BAND, TOL_GRAD, TOL_O, TOL_TSTAT, bf16_to_f64, bwd_decision_check, check_rows,
                          decision_report, legal_mask, nesting_check, rel_l2, tstat_report)

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mass_gated_sparse_amd import ops as _ops
    return _ops


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _rows(blocks, bq, L):
    return np.concatenate([np.arange(b * bq, min(b * bq + bq, L)) for b in blocks])


@functools.lru_cache(maxsize=2)
def _inputs(name, family):
    """Seeded inputs of a workload (host bf16 arrays and their fp64 values),
    shared by the tau values of one family."""
    w = WORKLOADS[name]
    x = prefill_inputs(w, family=family)
    xf = {n: to_f64(x[n], w.dtype) for n in ("q", "k", "v", "do")}
    return x, xf


def _prefill_full(ops, name, tau, qblocks, ktiles, family="planted"):
    w = WORKLOADS[name]
    x, xf = _inputs(name, family)
    q, k, v, do = (_dev(x[n]) for n in ("q", "k", "v", "do"))
    bq, bk = w.bq, w.bk
    o, lse, st = ops.fwd(q, k, v, tau, tile=(bq, bk), stats=True)
    dq, dk, dv, stb = ops.bwd(q, k, v, o, lse, do, tau, tile=(bq, bk), stats=True)
    torch.cuda.synchronize()
    B, H, L, d = q.shape
    nt = -(-L // bk)
    legal = legal_mask(L, bq, bk)
    gk = ops.bits_to_keep(st["keep_bits"], nt)
    gkb = ops.bits_to_keep(stb["keep_bits"], nt)
    gkb2 = ops.bits_to_keep(stb["keep_bits_dkdv"], nt)
    assert (gkb[..., legal] == gkb2[..., legal]).all()
    ts, tsb = st["test_stat"].cpu().numpy(), stb["test_stat"].cpu().numpy()
    qf, kf, vf, dof = (xf[n] for n in ("q", "k", "v", "do"))
    sq = list(qblocks)
    what = f"{name}/{family} tau={tau}"
    # forward, sampled query blocks (replay only on band tiles)
    oo, ol, ok, oT, rs = oracle.fwd(qf, kf, vf, tau, bq, bk, replay=gk, band=BAND, qblocks=qblocks, scales=True)
    sel = np.zeros_like(legal)
    sel[sq] = legal[sq]
    bad, near, _ = decision_report(gk, ok, oT, sel, what="fwd " + what, gpu_ts=ts)
    assert bad == 0, f"{what}: {bad} forward decisions differ"
    worst, nbad = tstat_report(ts, oT, sel, tau)
    assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
    assert (st["kept"].cpu().numpy()[:, :, sq] == (ok * legal).sum(-1)[:, :, sq]).all()
    rows = _rows(qblocks, bq, L)
    of = bf16_to_f64(o)
    assert rel_l2(of[:, :, rows], oo[:, :, rows]) <= TOL_O
    assert np.abs(lse.cpu().numpy()[:, :, rows] - ol[:, :, rows]).max() <= 1e-3
    check_rows("o", of[:, :, rows], oo[:, :, rows], what, r=rs[:, :, rows])
    # backward against the GPU's own forward state, sampled blocks and key
    # tiles, free-running oracle: decisions and kept counts bit-identical
    lf = lse.cpu().numpy().astype(np.float64)
    gq, gkk, gv, okb, oTb, sc = oracle.bwd(qf, kf, vf, of, lf, dof, tau, bq, bk, qblocks=qblocks, ktiles=ktiles,
                                           scales=True)
    selb = sel.copy()
    for t in ktiles:
        selb[:, t] |= legal[:, t]
    bwd_decision_check(gkb, okb, oTb, selb, what="bwd " + what, gpu_ts=tsb)
    worst, nbad = tstat_report(tsb, oTb, selb, tau)
    assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
    assert (stb["kept"].cpu().numpy()[:, :, sq] == (okb * legal).sum(-1)[:, :, sq]).all()
    krows = _rows(ktiles, bk, L)
    pairs = (("dq", bf16_to_f64(dq)[:, :, rows], gq[:, :, rows], sc["rq"][:, :, rows], sc["cq"][:, :, rows]),
             ("dk", bf16_to_f64(dk)[:, :, krows], gkk[:, :, krows], sc["rk"][:, :, krows], sc["ck"][:, :, krows]),
             ("dv", bf16_to_f64(dv)[:, :, krows], gv[:, :, krows], sc["rv"][:, :, krows], None))
    e = [rel_l2(a, b) for _, a, b, _, _ in pairs]
    assert max(e) <= TOL_GRAD, e
    for n, a, b, r, c in pairs:
        check_rows(n, a, b, what, r=r, c=c)
    # backward support nested in forward's, on the GPU's decisions over every legal tile
    nesting_check(gk, gkb, legal, ts, tsb, what)
    if tau == 0.0:
        assert gk[..., legal].all() and gkb[..., legal].all()
    return legal, gk, gkb


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_train128k_full(ops, tau):
    _prefill_full(ops, "train128k", tau, qblocks=(0, 1, 300, 1023), ktiles=(0, 1, 1500, 2046, 2047))


def test_chunk16k_full(ops):
    """Chunked prefill in the bench's configuration: the last 16,384 rows of
    the 128K training shape as one chunk at key offset 114,688 against the
    131,072-key cache, tau=1, on sampled query blocks of the chunk."""
    w = WORKLOADS["train128k"]
    P, Lq = w.L - 16384, 16384
    x, xf = _inputs("train128k", "planted")
    qc = np.ascontiguousarray(x["q"][:, :, P:])
    q, k, v = _dev(qc), _dev(x["k"]), _dev(x["v"])
    o, lse, st = ops.fwd_chunk(q, k, v, P, 1.0, stats=True)
    torch.cuda.synchronize()
    nt = -(-(P + Lq) // w.bk)
    gk = ops.bits_to_keep(st["keep_bits"], nt)
    qblocks = (0, 63, 127)
    qf, kf, vf = to_f64(qc, "bf16"), xf["k"], xf["v"]
    oo, ol, ok, oT, rs = oracle.fwd_chunk(qf, kf, vf, P, 1.0, w.bq, w.bk, replay=gk, band=BAND, qblocks=qblocks,
                                          scales=True)
    from tests.parity import chunk_legal_mask
    legal = chunk_legal_mask(Lq, P, w.bq, w.bk)
    sel = np.zeros_like(legal)
    sel[list(qblocks)] = legal[list(qblocks)]
    ts = st["test_stat"].cpu().numpy()
    bad, near, _ = decision_report(gk, ok, oT, sel, what="chunk16k tau=1", gpu_ts=ts)
    assert bad == 0, f"{bad} chunk decisions differ"
    worst, nbad = tstat_report(ts, oT, sel, 1.0)
    assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
    assert (st["kept"].cpu().numpy()[:, :, list(qblocks)] == (ok * legal).sum(-1)[:, :, list(qblocks)]).all()
    rows = _rows(qblocks, w.bq, Lq)
    assert rel_l2(bf16_to_f64(o)[:, :, rows], oo[:, :, rows]) <= TOL_O
    assert np.abs(lse.cpu().numpy()[:, :, rows] - ol[:, :, rows]).max() <= 1e-3
    check_rows("o", bf16_to_f64(o)[:, :, rows], oo[:, :, rows], "chunk16k tau=1", r=rs[:, :, rows])


@pytest.mark.parametrize("tau", [0.0, 0.5, 1.0, 2.0])
@pytest.mark.parametrize("family", ["planted", "planted_c1", "diffuse"])
def test_sweep32k_full(ops, tau, family):
    """Every (family, tau) the 32K sweep times, including the ungated
    instantiation at tau = 0."""
    _prefill_full(ops, "sweep32k", tau, qblocks=(0, 77, 255), ktiles=(0, 300, 510, 511), family=family)


def test_mw8k_full(ops):
    legal, gk, gkb = _prefill_full(ops, "mw8k", 1.0, qblocks=(0, 5, 40, 63), ktiles=(0, 64, 126, 127))
    kept = gk[..., legal].mean()
    assert 0.0 < kept < 1.0


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_gqa8k_full(ops, tau):
    """Grouped K/V heads at 8K (8 query heads over 2 K/V heads)."""
    _prefill_full(ops, "gqa8k", tau, qblocks=(0, 21, 63), ktiles=(0, 70, 127))


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_decode128k_full(ops, tau):
    w = WORKLOADS["decode128k"]
    x = decode_inputs(w, threads=16)
    q, kc, vc = (_dev(x[n]) for n in ("q", "k", "v"))
    o, lse, st = ops.decode(q, kc, vc, w.L, tau, split_keys=w.split_keys, bk=w.bk, stats=True)
    torch.cuda.synchronize()
    tps = w.split_keys // w.bk
    gk = ops.bits_to_keep(st["keep_bits"], tps)
    ts = st["test_stat"].cpu().numpy()
    nsplit = -(-w.L // w.split_keys)
    legal = np.zeros((nsplit, tps), bool)
    for p in range(nsplit):
        legal[p, : -(-(min((p + 1) * w.split_keys, w.L) - p * w.split_keys) // w.bk)] = True
    og, lg = bf16_to_f64(o), lse.cpu().numpy()
    for b, g in [(0, 0), (7, 3), (15, 7)]:
        hs = slice(g * w.group, (g + 1) * w.group)
        qs = to_f64(x["q"][b:b + 1, hs], "bf16")
        ks = to_f64(x["k"][b:b + 1, g:g + 1], "bf16")
        vs = to_f64(x["v"][b:b + 1, g:g + 1], "bf16")
        oo, ol, ok, oT = oracle.decode(qs, ks, vs, w.L, tau, w.split_keys, w.bk,
                                       replay=gk[b:b + 1, g:g + 1, None], band=BAND)
        what = f"decode128k tau={tau} (b={b}, g={g})"
        bad, near, _ = decision_report(gk[b, g], ok[0, 0, 0], oT[0, 0, 0], legal, what=what, gpu_ts=ts[b, g])
        assert bad == 0
        worst, nbad = tstat_report(ts[b, g], oT[0, 0, 0], legal, tau)
        assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
        assert (st["kept"].cpu().numpy()[b, g] == (ok[0, 0, 0] * legal).sum(-1)).all()
        assert rel_l2(og[b, hs], oo[0]) <= TOL_O
        assert np.abs(lg[b, hs] - ol[0]).max() <= 1e-3
        check_rows("o_decode", og[b, hs], oo[0], what)
    assert (st["legal"].cpu().numpy() == legal.sum(-1)).all()


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_decode128k_seeded_full(ops, tau):
    """Seeded decode at the full decode shape, sampled (sequence, KV head)
    groups against the oracle's seeded decode."""
    w = WORKLOADS["decode128k"]
    x = decode_inputs(w, threads=16)
    q, kc, vc = (_dev(x[n]) for n in ("q", "k", "v"))
    o, lse, st = ops.decode(q, kc, vc, w.L, tau, split_keys=w.split_keys, bk=w.bk, stats=True, seeded=True)
    torch.cuda.synchronize()
    nsplit, tps = oracle.seeded_decode_shapes(w.L, w.split_keys, w.bk)
    gk = ops.bits_to_keep(st["keep_bits"], tps)
    ts = st["test_stat"].cpu().numpy()
    jd = (w.L - 1) // w.bk
    legal = np.zeros((nsplit, tps), bool)
    for p in range(nsplit):
        hi = jd - p * tps
        legal[p, : hi - max(0, hi - tps + 1) + 1] = True
    og, lg = bf16_to_f64(o), lse.cpu().numpy()
    for b, g in [(0, 0), (7, 3), (15, 7)]:
        hs = slice(g * w.group, (g + 1) * w.group)
        qs = to_f64(x["q"][b:b + 1, hs], "bf16")
        ks = to_f64(x["k"][b:b + 1, g:g + 1], "bf16")
        vs = to_f64(x["v"][b:b + 1, g:g + 1], "bf16")
        oo, ol, ok, oT = oracle.decode_seeded(qs, ks, vs, w.L, tau, w.split_keys, w.bk,
                                              replay=gk[b:b + 1, g:g + 1, None], band=BAND)
        what = f"seeded decode128k tau={tau} (b={b}, g={g})"
        bad, near, _ = decision_report(gk[b, g], ok[0, 0, 0], oT[0, 0, 0], legal, what=what, gpu_ts=ts[b, g])
        assert bad == 0
        worst, nbad = tstat_report(ts[b, g], oT[0, 0, 0], legal, tau)
        assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
        assert (st["kept"].cpu().numpy()[b, g] == (ok[0, 0, 0] * legal).sum(-1)).all()
        assert rel_l2(og[b, hs], oo[0]) <= TOL_O
        assert np.abs(lg[b, hs] - ol[0]).max() <= 1e-3
        check_rows("o_decode", og[b, hs], oo[0], what)
    assert (st["legal"].cpu().numpy() == legal.sum(-1)).all()


@pytest.mark.parametrize("seeded", [False, True])
def test_decode128k_per_head_votes_full(ops, seeded):
    """The full decode shape with one vote per query head (rows_per_vote = 1),
    tau = 1, plain and seeded: sampled (sequence, KV head) groups against the
    oracle with the same vote groups."""
    w = WORKLOADS["decode128k"]
    x = decode_inputs(w, threads=16)
    q, kc, vc = (_dev(x[n]) for n in ("q", "k", "v"))
    o, lse, st = ops.decode(q, kc, vc, w.L, 1.0, split_keys=w.split_keys, bk=w.bk, stats=True, seeded=seeded,
                            rows_per_vote=1)
    torch.cuda.synchronize()
    G = w.group
    if seeded:
        nsplit, tps = oracle.seeded_decode_shapes(w.L, w.split_keys, w.bk)
        jd = (w.L - 1) // w.bk
        legal = np.zeros((nsplit, tps), bool)
        for p in range(nsplit):
            hi = jd - p * tps
            legal[p, : hi - max(0, hi - tps + 1) + 1] = True
        ref = oracle.decode_seeded
    else:
        nsplit, tps = -(-w.L // w.split_keys), w.split_keys // w.bk
        legal = np.zeros((nsplit, tps), bool)
        for p in range(nsplit):
            legal[p, : -(-(min((p + 1) * w.split_keys, w.L) - p * w.split_keys) // w.bk)] = True
        ref = oracle.decode
    gk = ops.bits_to_keep(st["keep_bits"], tps)  # [B, Hq, nsplit, tps]: one vote group per query head
    assert gk.shape == (w.B, w.H, nsplit, tps)
    og, lg = bf16_to_f64(o), lse.cpu().numpy()
    for b, g in [(0, 0), (9, 5), (15, 7)]:
        hs = slice(g * G, (g + 1) * G)
        qs = to_f64(x["q"][b:b + 1, hs], "bf16")
        ks = to_f64(x["k"][b:b + 1, g:g + 1], "bf16")
        vs = to_f64(x["v"][b:b + 1, g:g + 1], "bf16")
        oo, ol, ok, oT = ref(qs, ks, vs, w.L, 1.0, w.split_keys, w.bk, rows_per_vote=1,
                             replay=gk[b:b + 1, hs][:, None], band=BAND)
        what = f"decode128k per-head votes seeded={seeded} (b={b}, g={g})"
        bad, near, _ = decision_report(gk[b, hs], ok[0, 0], oT[0, 0], legal, what=what,
                                       gpu_ts=st["test_stat"].cpu().numpy()[b, hs])
        assert bad == 0
        assert (st["kept"].cpu().numpy()[b, hs] == (ok[0, 0] * legal).sum(-1)).all()
        assert rel_l2(og[b, hs], oo[0]) <= TOL_O
        assert np.abs(lg[b, hs] - ol[0]).max() <= 1e-3
        check_rows("o_decode", og[b, hs], oo[0], what)
    assert (st["legal"].cpu().numpy() == legal.sum(-1)).all()
    assert (st["kept"].cpu().numpy() == (gk * legal).sum(-1)).all()
