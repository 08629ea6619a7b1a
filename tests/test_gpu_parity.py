"""GPU parity: libmala.so (through its C ABI) against the fp64 CPU oracle.

Inputs are seeded instances of the named workloads (synth); the oracle runs
on exactly the values the GPU received.  Forward/decode decisions must match
tile for tile outside the |T-1| <= 1e-4 band (the oracle replays the GPU's
decisions inside it, and the band tiles are printed); backward decisions must
match the free-running oracle tile for tile given the GPU's own O and lse, and
kept counts must equal the oracle's; O within rel-L2 5e-3, gradients within
1e-2 over the tensor, and every row within the per-row bounds of
tests/parity.py.
"""
import math

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, prefill_inputs, decode_inputs, round_to, to_f64
from tests.parity import (BAND, TOL_GRAD, TOL_O, TOL_TSTAT, bf16_to_f64, bwd_decision_check, check_rows,
                          chunk_legal_mask, decision_report, legal_mask, rel_l2, tstat_report)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dev_tensors(x, dtype, names):
    out = []
    for n in names:
        a = x[n]
        if dtype == "bf16":
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        out.append(t.cuda().contiguous())
    return out


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mass_gated_sparse_amd import ops as _ops
    return _ops


def _prefill_case(name, L, heads, family="planted"):
    w = WORKLOADS[name]
    x = prefill_inputs(w, family=family, L=L, heads=heads)
    for n in x:
        x[n] = np.ascontiguousarray(x[n][:, list(heads)])
    return w, x


def _check_fwd(ops, w, x, tau, bq, bk):
    q, k, v = _dev_tensors(x, w.dtype, ("q", "k", "v"))
    o, lse, st = ops.fwd(q, k, v, tau, tile=(bq, bk), stats=True)
    torch.cuda.synchronize()
    B, H, L, d = q.shape
    nt = -(-L // bk)
    gk = ops.bits_to_keep(st["keep_bits"], nt)
    qf, kf, vf = (to_f64(x[n], w.dtype) for n in ("q", "k", "v"))
    oo, ol, ok, oT, rs = oracle.fwd(qf, kf, vf, tau, bq, bk, replay=gk, band=BAND, scales=True)
    legal = legal_mask(L, bq, bk)
    what = f"fwd L={L} tau={tau}"
    ts = st["test_stat"].cpu().numpy() if "test_stat" in st else None
    bad, near, near_list = decision_report(gk, ok, oT, legal, what=what, gpu_ts=ts)
    assert bad == 0, f"forward decisions differ outside the band on {bad} tiles"
    kept = st["kept"].cpu().numpy()
    assert (kept == (gk * legal).sum(-1)).all()
    assert (kept == (ok * legal).sum(-1)).all(), "kept counts differ from the oracle's"
    assert (st["legal"].cpu().numpy() == legal.sum(-1)[None, None, :]).all()
    e_o = rel_l2(bf16_to_f64(o), oo)
    e_l = float(np.abs(lse.cpu().numpy() - ol).max())
    assert e_o <= TOL_O, e_o
    assert e_l <= 1e-3, e_l
    check_rows("o", bf16_to_f64(o), oo, what, r=rs)
    if "test_stat" in st:  # the GPU's own test statistic, tile by tile
        worst, nbad = tstat_report(st["test_stat"].cpu().numpy(), oT, legal, tau)
        assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
    return dict(o=o, lse=lse, keep=gk, T=oT, near=near, err_o=e_o, legal=legal)


@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0, 16.0, math.inf])
def test_fwd_f32_tiny(ops, tau):
    w, x = _prefill_case("tiny", None, range(2))
    r = _check_fwd(ops, w, x, tau, 64, 64)
    assert r["err_o"] < 1e-5


@pytest.mark.parametrize("L,heads", [(1000, (0, 2, 5)), (2048, (1, 3, 6, 9))])
@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0, math.inf])
def test_fwd_bf16(ops, L, heads, tau):
    w, x = _prefill_case("mw8k", L, heads)
    r = _check_fwd(ops, w, x, tau, 128, 64)
    if tau == 4.0:
        assert (r["keep"][..., r["legal"]] == 0).any()  # gating exercised


def _check_bwd(ops, w, x, tau, bq, bk):
    q, k, v, do = _dev_tensors(x, w.dtype, ("q", "k", "v", "do"))
    o, lse = ops.fwd(q, k, v, tau, tile=(bq, bk))
    dq, dk, dv, st = ops.bwd(q, k, v, o, lse, do, tau, tile=(bq, bk), stats=True)
    torch.cuda.synchronize()
    B, H, L, d = q.shape
    nt = -(-L // bk)
    gk = ops.bits_to_keep(st["keep_bits"], nt)
    gk2 = ops.bits_to_keep(st["keep_bits_dkdv"], nt)
    legal = legal_mask(L, bq, bk)
    assert (gk[..., legal] == gk2[..., legal]).all(), "dQ and dK/dV passes disagree"
    qf, kf, vf, dof = (to_f64(x[n], w.dtype) for n in ("q", "k", "v", "do"))
    of, lf = bf16_to_f64(o), lse.cpu().numpy().astype(np.float64)
    # the free-running oracle (no replay): backward decisions must be bit-identical
    gq, gkk, gv, ok, oT, sc = oracle.bwd(qf, kf, vf, of, lf, dof, tau, bq, bk, scales=True)
    what = f"bwd L={L} tau={tau}"
    ts = st["test_stat"].cpu().numpy() if "test_stat" in st else None
    near = bwd_decision_check(gk, ok, oT, legal, what=what, gpu_ts=ts)
    assert (st["kept"].cpu().numpy() == (ok * legal).sum(-1)).all(), "kept counts differ from the oracle's"
    assert (st["kept"].cpu().numpy() == (gk * legal).sum(-1)).all()
    if ts is not None:
        worst, nbad = tstat_report(ts, oT, legal, tau)
        assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
    errs = [rel_l2(bf16_to_f64(a), b) for a, b in ((dq, gq), (dk, gkk), (dv, gv))]
    if tau == math.inf:
        assert all(float(t.abs().max()) == 0.0 for t in (dq, dk, dv))
    else:
        assert max(errs) <= TOL_GRAD, errs
        check_rows("dq", bf16_to_f64(dq), gq, what, r=sc["rq"], c=sc["cq"])
        check_rows("dk", bf16_to_f64(dk), gkk, what, r=sc["rk"], c=sc["ck"])
        check_rows("dv", bf16_to_f64(dv), gv, what, r=sc["rv"])
    return dict(keep=gk, errs=errs, near=near)


@pytest.mark.parametrize("tau", [0.0, 1.0, 16.0, math.inf])
def test_bwd_f32_tiny(ops, tau):
    w, x = _prefill_case("tiny", None, range(2))
    r = _check_bwd(ops, w, x, tau, 64, 64)
    if tau not in (math.inf,):
        assert max(r["errs"]) < 1e-5


@pytest.mark.parametrize("L,heads", [(1000, (0, 2, 5)), (2048, (1, 3))])
@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0, math.inf])
def test_bwd_bf16(ops, L, heads, tau):
    w, x = _prefill_case("mw8k", L, heads)
    _check_bwd(ops, w, x, tau, 128, 64)


@pytest.mark.parametrize("L,H,Hkv", [(1000, 64, 64), (900, 64, 64), (2048, 64, 32)])
@pytest.mark.parametrize("tau", [0.0, 1.0, math.inf])
def test_bwd_pair_layout_bf16(ops, L, H, Hkv, tau):
    """dK/dV in the tile-pair layout, which the launcher takes when
    B * Hkv * ceil(L/128) >= 512 (every case here): ragged lengths whose last
    pair has no second tile and whose last block has no second 64-row half
    (L=900), a ragged last block with both (L=1000), and grouped K/V heads.
    Decisions of both passes, and dQ/dK/dV against the oracle on sampled
    query blocks and key tiles, the last ones included."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["mw8k"], H=H, Hkv=Hkv)
    nqb, nt = -(-L // 128), -(-L // 64)
    assert nqb * Hkv >= 512
    x = prefill_inputs(w, L=L)
    q, k, v, do = _dev_tensors(x, "bf16", ("q", "k", "v", "do"))
    o, lse = ops.fwd(q, k, v, tau)
    dq, dk, dv, st = ops.bwd(q, k, v, o, lse, do, tau, stats=True)
    torch.cuda.synchronize()
    gk = ops.bits_to_keep(st["keep_bits"], nt)
    gk2 = ops.bits_to_keep(st["keep_bits_dkdv"], nt)
    legal = legal_mask(L, 128, 64)
    assert (gk[..., legal] == gk2[..., legal]).all(), "dQ and dK/dV passes disagree"
    if tau == math.inf:
        assert all(float(t.abs().max()) == 0.0 for t in (dq, dk, dv))
        return
    qblocks, ktiles = (0, nqb // 2, nqb - 1), (0, 1, nt // 2, nt - 2, nt - 1)
    qf, kf, vf, dof = (to_f64(x[n], "bf16") for n in ("q", "k", "v", "do"))
    of, lf = bf16_to_f64(o), lse.cpu().numpy().astype(np.float64)
    gq, gkk, gv, okb, oTb, sc = oracle.bwd(qf, kf, vf, of, lf, dof, tau, 128, 64, qblocks=qblocks, ktiles=ktiles,
                                           scales=True)
    sel = np.zeros_like(legal)
    sel[list(qblocks)] = legal[list(qblocks)]
    for t in ktiles:
        sel[:, t] |= legal[:, t]
    what = f"bwd pairs L={L} H={H} Hkv={Hkv} tau={tau}"
    bwd_decision_check(gk, okb, oTb, sel, what=what)
    sq = list(qblocks)
    assert (st["kept"].cpu().numpy()[:, :, sq] == (okb * legal).sum(-1)[:, :, sq]).all()
    rows = np.concatenate([np.arange(b * 128, min(b * 128 + 128, L)) for b in qblocks])
    krows = np.concatenate([np.arange(t * 64, min(t * 64 + 64, L)) for t in ktiles])
    pairs = (("dq", bf16_to_f64(dq)[:, :, rows], gq[:, :, rows], sc["rq"][:, :, rows], sc["cq"][:, :, rows]),
             ("dk", bf16_to_f64(dk)[:, :, krows], gkk[:, :, krows], sc["rk"][:, :, krows], sc["ck"][:, :, krows]),
             ("dv", bf16_to_f64(dv)[:, :, krows], gv[:, :, krows], sc["rv"][:, :, krows], None))
    e = [rel_l2(a, b) for _, a, b, _, _ in pairs]
    assert max(e) <= TOL_GRAD, e
    for n, a, b, r, c in pairs:
        check_rows(n, a, b, what, r=r, c=c)


@pytest.mark.parametrize("L", [1000, 2048])
@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0, math.inf])
def test_gqa_bf16(ops, L, tau):
    """Grouped K/V heads (8 query heads over 2 K/V heads): forward decisions
    and O per query head, backward decisions per query head, dK/dV summed
    over each group."""
    w = WORKLOADS["gqa8k"]
    x = prefill_inputs(w, L=L)
    assert x["k"].shape[1] == 2 and x["q"].shape[1] == 8
    _check_fwd(ops, w, x, tau, 128, 64)
    _check_bwd(ops, w, x, tau, 128, 64)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 130, 200])
@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0])
def test_short_ragged_bf16(ops, L, tau):
    """Sequences shorter than one or two query blocks, ragged in the last tile."""
    w, x = _prefill_case("mw8k", L, (0, 3))
    _check_fwd(ops, w, x, tau, 128, 64)
    _check_bwd(ops, w, x, tau, 128, 64)


@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0])
def test_mqa_bf16(ops, tau):
    """Eight query heads over a single K/V head (multi-query attention)."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["gqa8k"], Hkv=1)
    x = prefill_inputs(w, L=700)
    assert x["k"].shape[1] == 1 and x["q"].shape[1] == 8
    _check_fwd(ops, w, x, tau, 128, 64)
    _check_bwd(ops, w, x, tau, 128, 64)


@pytest.mark.parametrize("tau,family", [(0.0, "planted"), (1.0, "planted"), (0.0, "diffuse")])
def test_autograd_wrapper(ops, tau, family):
    """mala_attention's autograd gradients are the mala_bwd gradients against
    its own forward state, bit for bit.  On diffuse inputs at tau=0 they also
    match a float32 dense attention reference (CPU autograd) within the
    backward tolerance.  (Not on planted inputs: their nearly one-hot rows make
    dS = P (dP - D) a cancellation, and the bf16 rounding of O inside D alone
    moves the exact dQ by about 1.2% there.)"""
    w = WORKLOADS["gqa8k"]
    x = prefill_inputs(w, L=640, family=family)
    q, k, v, do = _dev_tensors(x, "bf16", ("q", "k", "v", "do"))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = ops.mala_attention(qa, ka, va, tau)
    o.backward(do)
    o2, lse2 = ops.fwd(q, k, v, tau)
    dq, dk, dv = ops.bwd(q, k, v, o2, lse2, do, tau)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for g, r in ((qa.grad, dq), (ka.grad, dk), (va.grad, dv)):
        assert torch.equal(g, r)
    if family == "diffuse":
        qf, kf, vf, dof = (t.float().cpu() for t in (q, k, v, do))
        G = qf.shape[1] // kf.shape[1]
        qf.requires_grad_(True)
        kf.requires_grad_(True)
        vf.requires_grad_(True)
        kr, vr = kf.repeat_interleave(G, dim=1), vf.repeat_interleave(G, dim=1)
        s_ = (qf @ kr.transpose(-1, -2).contiguous()) / math.sqrt(qf.shape[-1])
        L = qf.shape[2]
        s_ = s_.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
        ref = torch.softmax(s_, dim=-1) @ vr
        ref.backward(dof)
        e_o = rel_l2(o.detach().float().cpu().numpy(), ref.detach().numpy())
        assert e_o <= TOL_O, e_o
        errs = [rel_l2(g.float().cpu().numpy(), r.numpy())
                for g, r in ((qa.grad, qf.grad), (ka.grad, kf.grad), (va.grad, vf.grad))]
        assert max(errs) <= TOL_GRAD, errs


@pytest.mark.parametrize("P,Lq,spare", [(0, 640, 0), (256, 300, 77), (333, 300, 0), (1000, 130, 64),
                                         (0, 1, 0), (511, 1, 0), (4095, 1, 1), (127, 129, 0), (64, 64, 0)])
@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0])
def test_fwd_chunk_bf16(ops, P, Lq, spare, tau):
    """Chunked prefill: a query chunk at key offset P against a K/V cache
    (grouped K/V heads, cache capacity beyond the valid keys), against the
    oracle's chunk forward; a block-aligned chunk also reproduces the
    whole-sequence forward's rows bit for bit."""
    w = WORKLOADS["gqa8k"]
    x = prefill_inputs(w, L=P + Lq)
    qx = np.ascontiguousarray(x["q"][:, :, P:])
    cache = {n: np.zeros(x[n].shape[:2] + (P + Lq + spare, w.d), x[n].dtype) for n in ("k", "v")}
    for n in ("k", "v"):
        cache[n][:, :, :P + Lq] = x[n]
    q = torch.from_numpy(qx.view(np.int16)).view(torch.bfloat16).cuda()
    kc, vc = (torch.from_numpy(cache[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("k", "v"))
    o, lse, st = ops.fwd_chunk(q, kc, vc, P, tau, stats=True)
    torch.cuda.synchronize()
    nt = -(-(P + Lq) // 64)
    gk = ops.bits_to_keep(st["keep_bits"], nt)
    qf = to_f64(qx, "bf16")
    kf, vf = (to_f64(x[n], "bf16") for n in ("k", "v"))
    oo, ol, ok, oT, rs = oracle.fwd_chunk(qf, kf, vf, P, tau, 128, 64, replay=gk, band=BAND, scales=True)
    legal = chunk_legal_mask(Lq, P, 128, 64)
    what = f"chunk P={P} Lq={Lq} tau={tau}"
    ts = st["test_stat"].cpu().numpy()
    bad, near, _ = decision_report(gk, ok, oT, legal, what=what, gpu_ts=ts)
    assert bad == 0, f"chunk decisions differ outside the band on {bad} tiles"
    worst, nbad = tstat_report(ts, oT, legal, tau)
    assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
    assert (st["kept"].cpu().numpy() == (gk * legal).sum(-1)).all()
    assert (st["kept"].cpu().numpy() == (ok * legal).sum(-1)).all()
    assert (st["legal"].cpu().numpy() == legal.sum(-1)[None, None, :]).all()
    assert rel_l2(bf16_to_f64(o), oo) <= TOL_O
    assert float(np.abs(lse.cpu().numpy() - ol).max()) <= 1e-3
    check_rows("o", bf16_to_f64(o), oo, what, r=rs)
    if P % 128 == 0:
        qa, ka, va = _dev_tensors(x, "bf16", ("q", "k", "v"))
        of, lf = ops.fwd(qa, ka, va, tau)
        torch.cuda.synchronize()
        assert torch.equal(o, of[:, :, P:]) and torch.equal(lse, lf[:, :, P:])


def _decode_case(Lk, batches, Lcap=None):
    w = WORKLOADS["decode128k"]
    x = decode_inputs(w, Lk=Lk, Lcap=Lcap, batches=batches)
    for n in x:
        x[n] = np.ascontiguousarray(x[n][list(batches)])
    return w, x


@pytest.mark.parametrize("Lk,split,Lcap", [(3000, 1024, None), (4097, 4096, 4200), (64, 4096, None), (1, 64, 100)])
@pytest.mark.parametrize("tau", [0.0, 1.0, 16.0, math.inf])
def test_decode_bf16(ops, Lk, split, Lcap, tau):
    w, x = _decode_case(Lk, (0, 1), Lcap)
    q, kc, vc = _dev_tensors(x, "bf16", ("q", "k", "v"))
    o, lse, st = ops.decode(q, kc, vc, Lk, tau, split_keys=split, bk=64, stats=True)
    torch.cuda.synchronize()
    tps = split // 64
    gk = ops.bits_to_keep(st["keep_bits"], tps)  # [B, Hkv, nsplit, tps]
    qf, kf, vf = (to_f64(x[n], "bf16") for n in ("q", "k", "v"))
    oo, ol, ok, oT = oracle.decode(qf, kf, vf, Lk, tau, split, 64, replay=gk[:, :, None], band=BAND)
    nsplit = -(-Lk // split)
    legal = np.zeros((nsplit, tps), bool)
    for p in range(nsplit):
        legal[p, : -(-(min((p + 1) * split, Lk) - p * split) // 64)] = True
    what = f"decode Lk={Lk} split={split} tau={tau}"
    ts = st["test_stat"].cpu().numpy()
    bad, near, _ = decision_report(gk, ok[:, :, 0], oT[:, :, 0], legal, what=what, gpu_ts=ts)
    assert bad == 0
    assert (st["legal"].cpu().numpy() == legal.sum(-1)).all()
    assert (st["kept"].cpu().numpy() == (ok[:, :, 0] * legal).sum(-1)).all()
    assert rel_l2(bf16_to_f64(o), oo) <= TOL_O
    assert float(np.abs(lse.cpu().numpy() - ol).max()) <= 1e-3
    worst, nbad = tstat_report(ts, oT[:, :, 0], legal, tau)
    assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
    check_rows("o_decode", bf16_to_f64(o), oo, what)


def seeded_legal(Lk, split, bk=64):
    """[nsplit, tps] legal tiles of the seeded decode (partition 0 = newest)."""
    nsplit, tps = oracle.seeded_decode_shapes(Lk, split, bk)
    jd = (Lk - 1) // bk
    legal = np.zeros((nsplit, tps), bool)
    for p in range(nsplit):
        hi = jd - p * tps
        legal[p, : hi - max(0, hi - tps + 1) + 1] = True
    return legal


@pytest.mark.parametrize("Lk,split,Lcap", [(3000, 1024, None), (4097, 4096, 4200), (1536, 512, None),
                                           (5000, 512, 5003), (64, 4096, None), (1, 64, 100), (20000, 4096, None),
                                           (40000, 16384, None), (70000, 32768, None)])
@pytest.mark.parametrize("tau", [0.0, 1.0, 16.0, math.inf])
def test_decode_seeded_bf16(ops, Lk, split, Lcap, tau):
    """mala_decode_seeded against the oracle's seeded decode: decisions per
    partition (partition 0 the newest), O and lse; with one partition it is
    mala_decode bit for bit.  Newest partitions of up to 256 tiles are
    replayed from tile states (40000 / 16384: 256 tiles), longer ones walked
    tile by tile (70000 / 32768: 512 tiles)."""
    w, x = _decode_case(Lk, (0, 1), Lcap)
    q, kc, vc = _dev_tensors(x, "bf16", ("q", "k", "v"))
    o, lse, st = ops.decode(q, kc, vc, Lk, tau, split_keys=split, bk=64, stats=True, seeded=True)
    torch.cuda.synchronize()
    nsplit, tps = oracle.seeded_decode_shapes(Lk, split, 64)
    gk = ops.bits_to_keep(st["keep_bits"], tps)  # [B, Hkv, nsplit, tps]
    qf, kf, vf = (to_f64(x[n], "bf16") for n in ("q", "k", "v"))
    oo, ol, ok, oT = oracle.decode_seeded(qf, kf, vf, Lk, tau, split, 64, replay=gk[:, :, None], band=BAND)
    legal = seeded_legal(Lk, split)
    what = f"seeded decode Lk={Lk} split={split} tau={tau}"
    ts = st["test_stat"].cpu().numpy()
    bad, near, _ = decision_report(gk, ok[:, :, 0], oT[:, :, 0], legal, what=what, gpu_ts=ts)
    assert bad == 0
    worst, nbad = tstat_report(ts, oT[:, :, 0], legal, tau)
    assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
    assert (st["legal"].cpu().numpy() == legal.sum(-1)).all()
    assert (st["kept"].cpu().numpy() == (gk * legal).sum(-1)).all()
    assert (st["kept"].cpu().numpy() == (ok[:, :, 0] * legal).sum(-1)).all()
    assert rel_l2(bf16_to_f64(o), oo) <= TOL_O
    assert float(np.abs(lse.cpu().numpy() - ol).max()) <= 1e-3
    check_rows("o_decode", bf16_to_f64(o), oo, what)
    if nsplit == 1:
        o2, lse2 = ops.decode(q, kc, vc, Lk, tau, split_keys=split, bk=64)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("seeded", [False, True])
@pytest.mark.parametrize("tau", [0.0, 1.0])
def test_decode_lone_tile_dominates(ops, seeded, tau):
    """A partition of a single tile whose key carries nearly all of every
    row's softmax mass: plain decode's last partition holds only the newest
    key (Lk = 4097, split 4096), a seeded decode's oldest partition only
    tile 0 (the query is aligned with key 0 there).  Its V must reach the
    output: O and lse against the oracle, and O close to that key's V row."""
    rng = np.random.default_rng(20261204)
    B, Hq, Hkv, Lk, d, split = 2, 8, 2, 4097, 128, 4096
    G = Hq // Hkv
    k = rng.standard_normal((B, Hkv, Lk, d))
    v = rng.standard_normal((B, Hkv, Lk, d))
    j = 0 if seeded else Lk - 1
    q = 2.0 * np.repeat(k[:, :, j, :], G, axis=1) + 0.1 * rng.standard_normal((B, Hq, d))
    x = {"q": round_to(q, "bf16"), "k": round_to(k, "bf16"), "v": round_to(v, "bf16")}
    qd, kd, vd = _dev_tensors(x, "bf16", ("q", "k", "v"))
    o, lse, st = ops.decode(qd, kd, vd, Lk, tau, split_keys=split, bk=64, stats=True, seeded=seeded)
    torch.cuda.synchronize()
    qf, kf, vf = (to_f64(x[n], "bf16") for n in ("q", "k", "v"))
    if seeded:
        nsplit, tps = oracle.seeded_decode_shapes(Lk, split, 64)
        gk = ops.bits_to_keep(st["keep_bits"], tps)
        oo, ol, ok, oT = oracle.decode_seeded(qf, kf, vf, Lk, tau, split, 64, replay=gk[:, :, None], band=BAND)
    else:
        gk = ops.bits_to_keep(st["keep_bits"], split // 64)
        oo, ol, ok, oT = oracle.decode(qf, kf, vf, Lk, tau, split, 64, replay=gk[:, :, None], band=BAND)
    og = bf16_to_f64(o)
    assert rel_l2(og, oo) <= TOL_O
    assert float(np.abs(lse.cpu().numpy() - ol).max()) <= 1e-3
    check_rows("o_decode", og, oo, f"lone tile seeded={seeded} tau={tau}")
    vj = np.repeat(vf[:, :, j, :], G, axis=1)  # the dominant key's V row, per query head
    assert rel_l2(og, vj) <= 0.05


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (16, 2)])
@pytest.mark.parametrize("Lk,split", [(3000, 1024), (4097, 4096)])
@pytest.mark.parametrize("tau", [0.0, 1.0, 16.0])
@pytest.mark.parametrize("seeded", [False, True])
def test_decode_groups_bf16(ops, Hq, Hkv, Lk, split, tau, seeded):
    """Decode with 1, 2 and 8 query heads per K/V head (the vote rows of a
    tile), plain and seeded, against the oracle."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["decode128k"], B=2, H=Hq, Hkv=Hkv)
    x = decode_inputs(w, Lk=Lk)
    q, kc, vc = _dev_tensors(x, "bf16", ("q", "k", "v"))
    o, lse, st = ops.decode(q, kc, vc, Lk, tau, split_keys=split, bk=64, stats=True, seeded=seeded)
    torch.cuda.synchronize()
    qf, kf, vf = (to_f64(x[n], "bf16") for n in ("q", "k", "v"))
    if seeded:
        nsplit, tps = oracle.seeded_decode_shapes(Lk, split, 64)
        legal = seeded_legal(Lk, split)
        ref = oracle.decode_seeded
    else:
        nsplit, tps = -(-Lk // split), split // 64
        legal = np.zeros((nsplit, tps), bool)
        for p in range(nsplit):
            legal[p, : -(-(min((p + 1) * split, Lk) - p * split) // 64)] = True
        ref = oracle.decode
    gk = ops.bits_to_keep(st["keep_bits"], tps)
    oo, ol, ok, oT = ref(qf, kf, vf, Lk, tau, split, 64, replay=gk[:, :, None], band=BAND)
    what = f"decode groups Hq={Hq} Hkv={Hkv} Lk={Lk} seeded={seeded} tau={tau}"
    bad, near, _ = decision_report(gk, ok[:, :, 0], oT[:, :, 0], legal, what=what,
                                   gpu_ts=st["test_stat"].cpu().numpy())
    assert bad == 0
    assert (st["legal"].cpu().numpy() == legal.sum(-1)).all()
    assert (st["kept"].cpu().numpy() == (ok[:, :, 0] * legal).sum(-1)).all()
    assert rel_l2(bf16_to_f64(o), oo) <= TOL_O
    assert float(np.abs(lse.cpu().numpy() - ol).max()) <= 1e-3
    check_rows("o_decode", bf16_to_f64(o), oo, what)


@pytest.mark.parametrize("Hq,Hkv,rpv", [(32, 8, 1), (32, 8, 2), (16, 2, 1), (16, 2, 4)])
@pytest.mark.parametrize("Lk,split", [(3000, 1024), (4097, 4096), (65, 64), (1, 64)])
@pytest.mark.parametrize("tau", [0.0, 1.0, 16.0, math.inf])
@pytest.mark.parametrize("seeded", [False, True])
def test_decode_rows_per_vote_bf16(ops, Hq, Hkv, rpv, Lk, split, tau, seeded):
    """Votes over rows_per_vote query heads of a KV group (one vote per head
    when 1), plain and seeded, against the oracle with the same vote groups:
    decisions and kept counts per vote group, O and lse."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["decode128k"], B=2, H=Hq, Hkv=Hkv)
    x = decode_inputs(w, Lk=Lk)
    q, kc, vc = _dev_tensors(x, "bf16", ("q", "k", "v"))
    o, lse, st = ops.decode(q, kc, vc, Lk, tau, split_keys=split, bk=64, stats=True, seeded=seeded,
                            rows_per_vote=rpv)
    torch.cuda.synchronize()
    qf, kf, vf = (to_f64(x[n], "bf16") for n in ("q", "k", "v"))
    if seeded:
        nsplit, tps = oracle.seeded_decode_shapes(Lk, split, 64)
        legal = seeded_legal(Lk, split)
        ref = oracle.decode_seeded
    else:
        nsplit, tps = -(-Lk // split), split // 64
        legal = np.zeros((nsplit, tps), bool)
        for p in range(nsplit):
            legal[p, : -(-(min((p + 1) * split, Lk) - p * split) // 64)] = True
        ref = oracle.decode
    vg = (Hq // Hkv) // rpv
    gk = ops.bits_to_keep(st["keep_bits"], tps)  # [B, Hkv * vg, nsplit, tps]
    assert gk.shape == (2, Hkv * vg, nsplit, tps)
    oo, ol, ok, oT = ref(qf, kf, vf, Lk, tau, split, 64, rows_per_vote=rpv,
                         replay=gk.reshape(2, Hkv, vg, nsplit, tps), band=BAND)
    ok, oT = ok.reshape(gk.shape), oT.reshape(gk.shape)
    what = f"decode votes Hq={Hq} Hkv={Hkv} rpv={rpv} Lk={Lk} seeded={seeded} tau={tau}"
    ts = st["test_stat"].cpu().numpy()
    bad, near, _ = decision_report(gk, ok, oT, legal, what=what, gpu_ts=ts)
    assert bad == 0
    worst, nbad = tstat_report(ts, oT, legal, tau)
    assert nbad == 0 and worst <= TOL_TSTAT, (worst, nbad)
    assert (st["legal"].cpu().numpy() == legal.sum(-1)).all()
    assert (st["kept"].cpu().numpy() == (gk * legal).sum(-1)).all()
    assert (st["kept"].cpu().numpy() == (ok * legal).sum(-1)).all()
    assert rel_l2(bf16_to_f64(o), oo) <= TOL_O
    assert float(np.abs(lse.cpu().numpy() - ol).max()) <= 1e-3
    check_rows("o_decode", bf16_to_f64(o), oo, what)


@pytest.mark.parametrize("seeded", [False, True])
def test_decode_rows_per_vote_g_is_default(ops, seeded):
    """rows_per_vote = G is the default whole-group vote, bit for bit."""
    w, x = _decode_case(5000, (0, 1))
    q, kc, vc = _dev_tensors(x, "bf16", ("q", "k", "v"))
    a = ops.decode(q, kc, vc, 5000, 1.0, split_keys=1024, stats=True, seeded=seeded)
    b = ops.decode(q, kc, vc, 5000, 1.0, split_keys=1024, stats=True, seeded=seeded, rows_per_vote=w.group)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for n in ("kept", "legal", "keep_bits"):
        assert torch.equal(a[2][n], b[2][n]), n


def test_invalid_arguments_rejected(ops):
    from mass_gated_sparse_amd._lib import MalaError
    q = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MalaError):
        ops.fwd(q, q, q, -1.0)
    with pytest.raises(MalaError):
        ops.fwd(q, q, q, float("nan"))
    q64 = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MalaError) as e:
        ops.fwd(q64, q64, q64, 1.0)
    assert e.value.status == -2


def test_graph_capture_replays(ops):
    """The library only launches kernels on the caller's stream, so forward,
    backward (with the dK/dV statistics, which the call clears with a kernel)
    and both decodes can be captured in one HIP graph.  The graph is replayed
    several times, with other eager work and synchronizations between the
    replays, and every replay must equal the eager results bit for bit."""
    w, x = _prefill_case("mw8k", 1000, (0, 3))
    q, k, v, do = _dev_tensors(x, "bf16", ("q", "k", "v", "do"))
    o, lse = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = ops.bwd_workspace(q)
    st = ops.prefill_stats_buffers(q.shape[0], q.shape[1], 1000, (128, 64), q.device, dkdv=True)
    wd, xd = _decode_case(5000, (0, 1))
    qd, kc, vc = _dev_tensors(xd, "bf16", ("q", "k", "v"))
    od, ld = torch.empty_like(qd), torch.empty(qd.shape[:2], dtype=torch.float32, device="cuda")
    os_, ls_ = torch.empty_like(qd), torch.empty(qd.shape[:2], dtype=torch.float32, device="cuda")
    wsd = ops.decode_workspace(2, wd.H, wd.Hkv, 5000, wd.d, 1024, qd.device)
    wss = ops.decode_workspace(2, wd.H, wd.Hkv, 5000, wd.d, 1024, qd.device)

    def run():
        ops.fwd_into(q, k, v, o, lse, 1.0)
        ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, 1.0, ws, stats=st)
        ops.decode_into(qd, kc, vc, 5000, od, ld, 1.0, wsd, 1024)
        ops.decode_into(qd, kc, vc, 5000, os_, ls_, 1.0, wss, 1024, seeded=True)

    outs = (o, lse, dq, dk, dv, st["keep_bits"], st["keep_bits_dkdv"], od, ld, os_, ls_)
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on a side stream before capture
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for t in outs:
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {rep} differs"
