"""CPU oracle of MassAlloc Attention (MALA): ctypes wrapper of the fp64 C library.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the bench's
CPU-baseline leg import this package.  The GPU operator must never route
through it, and it imports nothing from the GPU package.

Inputs are fp64 numpy arrays (the exact values of the rounded bf16/fp32
inputs).  Layouts: prefill [B, H, L, d]; decode q [B, Hq, d] and caches
[B, Hkv, Lcap, d].  Decision arrays are uint8, statistics fp64 (T is NaN for
tiles not visited and for tau = 0).

The arithmetic lives in mala_oracle.c, whose header lists the passages it
follows and every reading of points the pages leave open.
"""
import ctypes
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .build import build, lib_path

_LIB = None
_D = ctypes.POINTER(ctypes.c_double)
_U8 = ctypes.POINTER(ctypes.c_uint8)
_L = ctypes.POINTER(ctypes.c_long)


def _lib():
    global _LIB
    if _LIB is None:
        p = lib_path()
        if not os.path.exists(p):
            build()
        lib = ctypes.CDLL(p)
        lib.oracle_fwd_head.argtypes = [_D, _D, _D, ctypes.c_long, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_int, ctypes.c_int, _L, ctypes.c_long, _U8, ctypes.c_double,
                                        _D, _D, _U8, _D, _D]
        lib.oracle_bwd_head.argtypes = [_D, _D, _D, _D, _D, _D, ctypes.c_long, ctypes.c_int, ctypes.c_double,
                                        ctypes.c_double, ctypes.c_int, ctypes.c_int, _L, ctypes.c_long, _L,
                                        ctypes.c_long, _U8, ctypes.c_double, _D, _D, _D, _U8, _D, _D]
        lib.oracle_decode_group.argtypes = [_D, ctypes.c_int, _D, _D, ctypes.c_long, ctypes.c_int, ctypes.c_double,
                                            ctypes.c_double, ctypes.c_long, ctypes.c_int, ctypes.c_int, _U8,
                                            ctypes.c_double, _D, _D, _U8, _D, _D, _D, _D]
        lib.oracle_decode_groups.argtypes = [ctypes.c_long, _D, ctypes.c_int, _D, _D, ctypes.c_long, ctypes.c_long,
                                             ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_long,
                                             ctypes.c_int, ctypes.c_int, _U8, ctypes.c_double, _D, _D, _U8, _D]
        lib.oracle_decode_seeded_group.argtypes = lib.oracle_decode_group.argtypes
        lib.oracle_decode_seeded_groups.argtypes = lib.oracle_decode_groups.argtypes
        lib.oracle_fwd_chunk_head.argtypes = [_D, _D, _D, ctypes.c_long, ctypes.c_long, ctypes.c_int,
                                              ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int, _L,
                                              ctypes.c_long, _U8, ctypes.c_double, _D, _D, _U8, _D, _D]
        for f in ("oracle_fwd_head", "oracle_bwd_head", "oracle_decode_group", "oracle_decode_groups",
                  "oracle_decode_seeded_group", "oracle_decode_seeded_groups", "oracle_fwd_chunk_head"):
            getattr(lib, f).restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _p(a, t):
    if a is None:
        return None
    return a.ctypes.data_as(t)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ids(x):
    if x is None:
        return None, 0
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int64).ravel()).astype(np.int_)
    return a, len(a)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def default_scale(d):
    return 1.0 / math.sqrt(d)


def _per_head(B, H, fn):
    """Run fn(b, h) for every head; heads run side by side (the C calls
    release the GIL; each call is independent)."""
    jobs = [(b, h) for b in range(B) for h in range(H)]
    if len(jobs) == 1:
        fn(*jobs[0])
        return
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        for f in [ex.submit(fn, b, h) for b, h in jobs]:
            f.result()


def _group(H, k):
    """Query heads per K/V head (grouped-query attention: q has H heads, k and
    v have Hkv; query head h attends with K/V head h // (H / Hkv))."""
    Hkv = k.shape[1]
    if H % Hkv:
        raise ValueError(f"H={H} is not a multiple of Hkv={Hkv}")
    return H // Hkv


def fwd(q, k, v, tau, bq, bk, scale=None, replay=None, band=1e-4, qblocks=None, scales=False):
    """MALA forward.  Returns (o, lse, keep, T); keep/T are [B, H, nqb, ntiles].
    q is [B, H, L, d]; k, v are [B, Hkv, L, d] with H % Hkv == 0.

    qblocks: optional iterable of query-block indices (same for every head);
    rows of other blocks are left NaN.
    replay: optional uint8 [B, H, nqb, ntiles] decisions adopted on tiles with
    |T - 1| <= band.
    scales: also return each row's error scale rs [B, H, L] (see
    oracle_fwd_head), for the parity tests' per-row bound.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    G = _group(H, k)
    scale = default_scale(d) if scale is None else float(scale)
    nqb, nt = -(-L // bq), -(-L // bk)
    o = np.full((B, H, L, d), np.nan)
    lse = np.full((B, H, L), np.nan)
    keep = np.zeros((B, H, nqb, nt), dtype=np.uint8)
    T = np.full((B, H, nqb, nt), np.nan)
    ids, n = _ids(qblocks)
    rp = None if replay is None else np.ascontiguousarray(replay, dtype=np.uint8)
    rs = np.full((B, H, L), np.nan) if scales else None

    def one(b, h):
        g = h // G  # the K/V head query head h reads
        rc = _lib().oracle_fwd_head(_p(q[b, h], _D), _p(k[b, g], _D), _p(v[b, g], _D), L, d, scale, float(tau),
                                    bq, bk, _p(ids, _L), n, _p(None if rp is None else rp[b, h], _U8),
                                    float(band), _p(o[b, h], _D), _p(lse[b, h], _D), _p(keep[b, h], _U8),
                                    _p(T[b, h], _D), _p(None if rs is None else rs[b, h], _D))
        _check(rc, "oracle_fwd_head")

    _per_head(B, H, one)
    return (o, lse, keep, T, rs) if scales else (o, lse, keep, T)


def fwd_chunk(q, k, v, p0, tau, bq, bk, scale=None, replay=None, band=1e-4, qblocks=None, scales=False):
    """MALA forward of a query chunk against a key cache (chunked prefill).

    q: [B, H, Lq, d], rows at key positions p0 .. p0 + Lq - 1; k, v:
    [B, Hkv, >= p0 + Lq, d] (the first p0 + Lq rows are the keys the chunk
    sees, its own included).  Row i has Lq_i = p0 + i + 1 visible keys.
    Returns (o, lse, keep, T); keep/T are [B, H, ceil(Lq/bq), ceil((p0+Lq)/bk)].
    qblocks: optional query-block indices of the chunk to compute (others
    left NaN / 0).  scales: also return the rows' error scales [B, H, Lq].
    """
    q = _f64(q)
    B, H, Lq, d = q.shape
    G = _group(H, k)
    Lk = int(p0) + Lq
    k, v = _f64(k[:, :, :Lk]), _f64(v[:, :, :Lk])
    scale = default_scale(d) if scale is None else float(scale)
    nqb, nt = -(-Lq // bq), -(-Lk // bk)
    o = np.full((B, H, Lq, d), np.nan)
    lse = np.full((B, H, Lq), np.nan)
    keep = np.zeros((B, H, nqb, nt), dtype=np.uint8)
    T = np.full((B, H, nqb, nt), np.nan)
    rp = None if replay is None else np.ascontiguousarray(replay, dtype=np.uint8)
    ids, n = _ids(qblocks)
    rs = np.full((B, H, Lq), np.nan) if scales else None

    def one(b, h):
        g = h // G
        rc = _lib().oracle_fwd_chunk_head(_p(q[b, h], _D), _p(k[b, g], _D), _p(v[b, g], _D), Lq, int(p0), d,
                                          scale, float(tau), bq, bk, _p(ids, _L), n,
                                          _p(None if rp is None else rp[b, h], _U8),
                                          float(band), _p(o[b, h], _D), _p(lse[b, h], _D), _p(keep[b, h], _U8),
                                          _p(T[b, h], _D), _p(None if rs is None else rs[b, h], _D))
        _check(rc, "oracle_fwd_chunk_head")

    _per_head(B, H, one)
    return (o, lse, keep, T, rs) if scales else (o, lse, keep, T)


def bwd(q, k, v, o, lse, do, tau, bq, bk, scale=None, replay=None, band=1e-4, qblocks=None, ktiles=None,
        scales=False):
    """MALA backward against the given forward state (o, lse).

    Returns (dq, dk, dv, keep, T).  qblocks / ktiles restrict which dq rows /
    dk,dv rows are computed (others NaN).  With grouped K/V heads
    (k, v: [B, Hkv, L, d]) every query head's contribution is computed with
    its shared K/V and dk, dv of a K/V head are the sum over its query heads
    (the gradient of a tensor used by several heads).
    scales: also return a dict of the rows' error scales (see oracle_bwd_head):
    "rq", "cq" [B, H, L] for dq rows; "rk", "ck", "rv" [B, Hkv, L] for dk and
    dv rows (root sum of squares over the query heads of a group).
    """
    q, k, v, o, lse, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(lse), _f64(do)
    B, H, L, d = q.shape
    G = _group(H, k)
    scale = default_scale(d) if scale is None else float(scale)
    nqb, nt = -(-L // bq), -(-L // bk)
    dq = np.full((B, H, L, d), np.nan)
    dk = np.full((B, H, L, d), np.nan)  # per query head; summed per group below
    dv = np.full((B, H, L, d), np.nan)
    keep = np.zeros((B, H, nqb, nt), dtype=np.uint8)
    T = np.full((B, H, nqb, nt), np.nan)
    qi, nq = _ids(qblocks)
    ki, nk = _ids(ktiles)
    rp = None if replay is None else np.ascontiguousarray(replay, dtype=np.uint8)
    es = np.full((B, H, 5, L), np.nan) if scales else None

    def one(b, h):
        g = h // G
        rc = _lib().oracle_bwd_head(_p(q[b, h], _D), _p(k[b, g], _D), _p(v[b, g], _D), _p(o[b, h], _D),
                                    _p(lse[b, h], _D), _p(do[b, h], _D), L, d, scale, float(tau), bq, bk,
                                    _p(qi, _L), nq, _p(ki, _L), nk, _p(None if rp is None else rp[b, h], _U8),
                                    float(band), _p(dq[b, h], _D), _p(dk[b, h], _D), _p(dv[b, h], _D),
                                    _p(keep[b, h], _U8), _p(T[b, h], _D), _p(None if es is None else es[b, h], _D))
        _check(rc, "oracle_bwd_head")

    _per_head(B, H, one)
    if G > 1:
        dk = dk.reshape(B, H // G, G, L, d).sum(axis=2)
        dv = dv.reshape(B, H // G, G, L, d).sum(axis=2)
    if not scales:
        return dq, dk, dv, keep, T
    kv = np.sqrt((es[:, :, 2:] ** 2).reshape(B, H // G, G, 3, L).sum(axis=2))
    sc = {"rq": es[:, :, 0], "cq": es[:, :, 1], "rk": kv[:, :, 0], "ck": kv[:, :, 1], "rv": kv[:, :, 2]}
    return dq, dk, dv, keep, T, sc


def decode_shapes(Lk, split_keys, bk):
    return -(-Lk // split_keys), -(-split_keys // bk)


def decode(q, kc, vc, Lk, tau, split_keys, bk, scale=None, rows_per_vote=None, replay=None, band=1e-4,
           units=None):
    """Split-KV MALA decode.  q [B, Hq, d]; kc, vc [B, Hkv, Lcap, d].

    Returns (o [B, Hq, d], lse [B, Hq], keep, T) with keep/T of shape
    [B, Hkv, G/rows_per_vote, nsplit, tps].  units: optional list of (b, g)
    pairs to compute (others left NaN / 0).
    """
    q = _f64(q)
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    R = G if rows_per_vote is None else int(rows_per_vote)
    scale = default_scale(d) if scale is None else float(scale)
    nsplit, tps = decode_shapes(Lk, split_keys, bk)
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    keep = np.zeros((B, Hkv, G // R, nsplit, tps), dtype=np.uint8)
    T = np.full((B, Hkv, G // R, nsplit, tps), np.nan)
    units = [(b, g) for b in range(B) for g in range(Hkv)] if units is None else list(units)
    n = len(units)
    qs = np.stack([q[b, g * G:(g + 1) * G] for b, g in units])
    ks = np.stack([_f64(kc[b, g, :Lk]) for b, g in units])
    vs = np.stack([_f64(vc[b, g, :Lk]) for b, g in units])
    ou = np.zeros((n, G, d))
    lu = np.zeros((n, G))
    kb = np.zeros((n, G // R, nsplit, tps), dtype=np.uint8)
    Tb = np.full((n, G // R, nsplit, tps), np.nan)
    rp = None
    if replay is not None:
        rp = np.ascontiguousarray(np.stack([replay[b, g] for b, g in units]), dtype=np.uint8)
    rc = _lib().oracle_decode_groups(n, _p(qs, _D), G, _p(ks, _D), _p(vs, _D), Lk * d, Lk, d, scale, float(tau),
                                     split_keys, bk, R, _p(rp, _U8), float(band), _p(ou, _D), _p(lu, _D),
                                     _p(kb, _U8), _p(Tb, _D))
    _check(rc, "oracle_decode_groups")
    for u, (b, g) in enumerate(units):
        o[b, g * G:(g + 1) * G] = ou[u]
        lse[b, g * G:(g + 1) * G] = lu[u]
        keep[b, g] = kb[u]
        T[b, g] = Tb[u]
    return o, lse, keep, T


def decode_group_partials(q, k, v, Lk, tau, split_keys, bk, scale=None, rows_per_vote=None):
    """One KV group (q [G, d], k/v [Lk, d]); also returns the per-partition
    states (m [G, nsplit], l [G, nsplit], acc [G, nsplit, d])."""
    q, k, v = _f64(q), _f64(k[:Lk]), _f64(v[:Lk])
    G, d = q.shape
    R = G if rows_per_vote is None else int(rows_per_vote)
    scale = default_scale(d) if scale is None else float(scale)
    nsplit, tps = decode_shapes(Lk, split_keys, bk)
    o = np.zeros((G, d)); lse = np.zeros(G)
    keep = np.zeros((G // R, nsplit, tps), dtype=np.uint8); T = np.full((G // R, nsplit, tps), np.nan)
    pm = np.zeros((G, nsplit)); pl = np.zeros((G, nsplit)); pa = np.zeros((G, nsplit, d))
    rc = _lib().oracle_decode_group(_p(q, _D), G, _p(k, _D), _p(v, _D), Lk, d, scale, float(tau), split_keys, bk,
                                    R, None, 0.0, _p(o, _D), _p(lse, _D), _p(keep, _U8), _p(T, _D),
                                    _p(pm, _D), _p(pl, _D), _p(pa, _D))
    _check(rc, "oracle_decode_group")
    return o, lse, keep, T, pm, pl, pa


def seeded_decode_shapes(Lk, split_keys, bk):
    """(nsplit, tps) of the seeded decode: partitions of split_keys/bk tiles
    counted back from the tile holding the newest key."""
    tps = split_keys // bk
    return -(-((Lk - 1) // bk + 1) // tps), tps


def decode_seeded(q, kc, vc, Lk, tau, split_keys, bk, scale=None, rows_per_vote=None, replay=None, band=1e-4,
                  units=None):
    """Split-KV MALA decode with seeded partitions (see
    oracle_decode_seeded_group): partition 0 holds the newest split_keys/bk
    tiles and starts empty; every older partition is tested against
    partition 0's final normalizer plus its own kept keys, with no forced
    keep.  Arguments and returns as decode(); keep/T are
    [B, Hkv, G/rows_per_vote, nsplit, tps] with partition 0 the newest."""
    q = _f64(q)
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    R = G if rows_per_vote is None else int(rows_per_vote)
    scale = default_scale(d) if scale is None else float(scale)
    if split_keys % bk:
        raise ValueError("split_keys must be a multiple of bk")
    nsplit, tps = seeded_decode_shapes(Lk, split_keys, bk)
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    keep = np.zeros((B, Hkv, G // R, nsplit, tps), dtype=np.uint8)
    T = np.full((B, Hkv, G // R, nsplit, tps), np.nan)
    units = [(b, g) for b in range(B) for g in range(Hkv)] if units is None else list(units)
    n = len(units)
    qs = np.stack([q[b, g * G:(g + 1) * G] for b, g in units])
    ks = np.stack([_f64(kc[b, g, :Lk]) for b, g in units])
    vs = np.stack([_f64(vc[b, g, :Lk]) for b, g in units])
    ou = np.zeros((n, G, d))
    lu = np.zeros((n, G))
    kb = np.zeros((n, G // R, nsplit, tps), dtype=np.uint8)
    Tb = np.full((n, G // R, nsplit, tps), np.nan)
    rp = None
    if replay is not None:
        rp = np.ascontiguousarray(np.stack([replay[b, g] for b, g in units]), dtype=np.uint8)
    rc = _lib().oracle_decode_seeded_groups(n, _p(qs, _D), G, _p(ks, _D), _p(vs, _D), Lk * d, Lk, d, scale,
                                            float(tau), split_keys, bk, R, _p(rp, _U8), float(band), _p(ou, _D),
                                            _p(lu, _D), _p(kb, _U8), _p(Tb, _D))
    _check(rc, "oracle_decode_seeded_groups")
    for u, (b, g) in enumerate(units):
        o[b, g * G:(g + 1) * G] = ou[u]
        lse[b, g * G:(g + 1) * G] = lu[u]
        keep[b, g] = kb[u]
        T[b, g] = Tb[u]
    return o, lse, keep, T


def decode_seeded_group_partials(q, k, v, Lk, tau, split_keys, bk, scale=None, rows_per_vote=None):
    """One KV group of the seeded decode (q [G, d], k/v [Lk, d]); also returns
    the partitions' own states (m [G, nsplit], l [G, nsplit], acc [G, nsplit, d])."""
    q, k, v = _f64(q), _f64(k[:Lk]), _f64(v[:Lk])
    G, d = q.shape
    R = G if rows_per_vote is None else int(rows_per_vote)
    scale = default_scale(d) if scale is None else float(scale)
    nsplit, tps = seeded_decode_shapes(Lk, split_keys, bk)
    o = np.zeros((G, d)); lse = np.zeros(G)
    keep = np.zeros((G // R, nsplit, tps), dtype=np.uint8); T = np.full((G // R, nsplit, tps), np.nan)
    pm = np.zeros((G, nsplit)); pl = np.zeros((G, nsplit)); pa = np.zeros((G, nsplit, d))
    rc = _lib().oracle_decode_seeded_group(_p(q, _D), G, _p(k, _D), _p(v, _D), Lk, d, scale, float(tau),
                                           split_keys, bk, R, None, 0.0, _p(o, _D), _p(lse, _D), _p(keep, _U8),
                                           _p(T, _D), _p(pm, _D), _p(pl, _D), _p(pa, _D))
    _check(rc, "oracle_decode_seeded_group")
    return o, lse, keep, T, pm, pl, pa
