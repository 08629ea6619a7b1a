"""Seeded synthetic inputs for MassAlloc Attention (MALA) workloads.

This module only draws and rounds inputs; it holds none of the operator's
arithmetic, and both the GPU path's tests and the CPU oracle consume what it
produces.

Structure.  The MALA digest's motivation paragraph says that on long contexts
the normalized attention mass concentrates on local windows, sink tokens and a
sparse retrieval set.  The planted family reproduces that structure by
building each query from keys of those three kinds plus noise:

    q_i = c_h * (0.3 z_i + 2.0 mean(k_0..k_3) + 1.5 k_{max(i - delta_i, 0)}
                 + 2.5 mean(k_{r_i1}, ..., k_{r_i4}))

with z_i ~ N(0, I), delta_i ~ U{0..31}, the r_ij drawn uniformly with
replacement from {0..i}, and a per-head sharpness multiplier c_h ~ U[lo, hi].
The planted_c1 family is the same recipe with c_h = 1 on every head (the
multiplier draw is skipped, every other draw is the planted family's).
K, V and dO rows are N(0, I).  The diffuse family draws Q and K i.i.d. N(0, I)
(near-uniform rows).  Everything is built in fp64 and rounded once to the
storage type: bf16 with round-to-nearest-even (kept as uint16 bit patterns),
or fp32.  The planted query uses the rounded keys, i.e. the values the
operator actually sees.

Reproducibility.  Every (tensor, batch, head) slice has its own PCG64 stream
seeded by SeedSequence(seed, spawn_key=(tensor, b, h)), so any slice can be
regenerated alone and the result does not depend on which slices were asked
for or in which order.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Workload

# stream ids of the per-slice generators
_K, _V, _DO, _Z, _DELTA, _RIDX, _MULT, _QDIFF = range(8)


def _rng(seed: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor, b, h))))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 to bf16 (round to nearest, ties to even) in one step.

    bf16 keeps 8 significant bits; fp64 has 53, so the low 45 bits of the
    fp64 pattern are rounded away.  The result is exactly representable in
    fp32, whose upper 16 bits are the bf16 pattern.  Finite normal inputs
    only (the generator never produces anything else).
    """
    b = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    f32 = r.view(np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array for fp64 values: uint16 bf16 patterns or float32."""
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values of a storage array produced by round_to."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def sharpness(w: Workload, b: int, h: int) -> float:
    if w.sharp_lo == w.sharp_hi:
        return float(w.sharp_lo)
    return float(_rng(w.seed, _MULT, b, h).uniform(w.sharp_lo, w.sharp_hi))


def _normal_rows(w: Workload, tensor: int, b: int, h: int, n: int) -> np.ndarray:
    return _rng(w.seed, tensor, b, h).standard_normal((n, w.d))


def _sink(kf: np.ndarray) -> np.ndarray:
    """Mean of the first four keys (of all keys when fewer exist)."""
    n = min(4, kf.shape[0])
    acc = kf[0].copy()
    for r in range(1, n):
        acc = acc + kf[r]
    return acc / n


def planted_query(w: Workload, b: int, h: int, kf: np.ndarray, positions: np.ndarray, c: float = None) -> np.ndarray:
    """fp64 planted queries for query head h at the given positions.

    kf: fp64 values of the (rounded) keys of head h's KV head, rows 0..max(positions).
    The noise, offsets, retrieval indices and multiplier come from head h's own
    streams; they are drawn for every position 0..max(positions) so that a
    position's query does not depend on which other positions are requested.
    `c` replaces the head's drawn multiplier when given.
    """
    n = int(positions.max()) + 1
    z = _rng(w.seed, _Z, b, h).standard_normal((n, w.d))
    delta = _rng(w.seed, _DELTA, b, h).integers(0, 32, size=n)
    hi = np.arange(1, n + 1, dtype=np.int64)[:, None]
    ridx = _rng(w.seed, _RIDX, b, h).integers(0, hi, size=(n, 4))
    c = sharpness(w, b, h) if c is None else float(c)
    i = positions.astype(np.int64)
    sink = _sink(kf)
    local = kf[np.maximum(i - delta[i], 0)]
    r = ridx[i]
    retr = (kf[r[:, 0]] + kf[r[:, 1]] + kf[r[:, 2]] + kf[r[:, 3]]) / 4.0
    return c * (0.3 * z[i] + 2.0 * sink[None, :] + 1.5 * local + 2.5 * retr)


def _decode_query(w: Workload, b: int, h: int, kf: np.ndarray, i: int) -> np.ndarray:
    """Planted query of head h at the single position i (same recipe as
    planted_query; the draws are made for that position only)."""
    z = _rng(w.seed, _Z, b, h).standard_normal(w.d)
    delta = int(_rng(w.seed, _DELTA, b, h).integers(0, 32))
    ridx = _rng(w.seed, _RIDX, b, h).integers(0, i + 1, size=4)
    c = sharpness(w, b, h)
    return c * (0.3 * z + 2.0 * _sink(kf) + 1.5 * kf[max(i - delta, 0)] + 2.5 * (kf[ridx[0]] + kf[ridx[1]] + kf[ridx[2]] + kf[ridx[3]]) / 4.0)


def prefill_inputs(w: Workload, family: str = "planted", L: int = None, heads=None):
    """Inputs of a prefill (fwd+bwd) workload.

    Returns dict with q, k, v, do of shape [B, H, L, d] in storage type
    (uint16 bf16 patterns or float32).  `L` overrides the workload's length
    (the streams are the workload's, so a shorter L is a different, still
    seeded instance).  `heads` restricts generation to those heads; the others
    stay zero.
    """
    if w.kind != "prefill":
        raise ValueError("prefill workload expected")
    L = w.L if L is None else int(L)
    heads = range(w.H) if heads is None else list(heads)
    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    out = {n: np.zeros((w.B, w.Hkv if n in ("k", "v") else w.H, L, w.d), dtype=sdt) for n in ("q", "k", "v", "do")}
    G = w.group
    for b in range(w.B):
        done_kv = set()
        for h in heads:
            g = h // G
            if g not in done_kv:
                out["k"][b, g] = round_to(_normal_rows(w, _K, b, g, L), w.dtype)
                out["v"][b, g] = round_to(_normal_rows(w, _V, b, g, L), w.dtype)
                done_kv.add(g)
            kf = to_f64(out["k"][b, g], w.dtype)
            if family == "planted":
                qf = planted_query(w, b, h, kf, np.arange(L))
            elif family == "planted_c1":
                qf = planted_query(w, b, h, kf, np.arange(L), c=1.0)
            elif family == "diffuse":
                qf = _normal_rows(w, _QDIFF, b, h, L)
            else:
                raise ValueError(family)
            out["q"][b, h] = round_to(qf, w.dtype)
            out["do"][b, h] = round_to(_normal_rows(w, _DO, b, h, L), w.dtype)
    return out


def decode_inputs(w: Workload, Lk: int = None, Lcap: int = None, batches=None, threads: int = 8):
    """Inputs of a decode workload.

    The cache of every (b, KV head) holds Lk keys/values (rows >= Lk up to
    Lcap stay zero); row Lk-1 is the new token's own key/value.  The query of
    every head is the planted query at position Lk-1.  Returns q [B, H, d],
    kcache and vcache [B, Hkv, Lcap, d] in storage type.
    """
    if w.kind != "decode":
        raise ValueError("decode workload expected")
    Lk = w.L if Lk is None else int(Lk)
    Lcap = Lk if Lcap is None else int(Lcap)
    if Lcap < Lk:
        raise ValueError("Lcap < Lk")
    batches = range(w.B) if batches is None else list(batches)
    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    q = np.zeros((w.B, w.H, w.d), dtype=sdt)
    kc = np.zeros((w.B, w.Hkv, Lcap, w.d), dtype=sdt)
    vc = np.zeros((w.B, w.Hkv, Lcap, w.d), dtype=sdt)
    G = w.group

    def one(bg):
        b, g = bg
        kc[b, g, :Lk] = round_to(_normal_rows(w, _K, b, g, Lk), w.dtype)
        vc[b, g, :Lk] = round_to(_normal_rows(w, _V, b, g, Lk), w.dtype)
        kf = to_f64(kc[b, g, :Lk], w.dtype)
        for h in range(g * G, (g + 1) * G):
            q[b, h] = round_to(_decode_query(w, b, h, kf, Lk - 1), w.dtype)

    work = [(b, g) for b in batches for g in range(w.Hkv)]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, work))
    return {"q": q, "k": kc, "v": vc}
