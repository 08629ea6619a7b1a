"""PyTorch-facing wrappers of the MALA C ABI (forward, backward, decode).

Tensors must be contiguous CUDA (HIP) tensors of dtype bfloat16 or float32.
Outputs and workspaces are allocated with torch (device memory plumbing);
the work itself is queued by libmala.so on torch's current stream.
"""
import ctypes
import math

import torch

from . import _lib
from ._lib import MALA_BF16, MALA_F32, Stats, Tile

DEFAULT_TILE = {torch.bfloat16: (128, 64), torch.float32: (64, 64)}


def _dt(t):
    if t.dtype == torch.bfloat16:
        return MALA_BF16
    if t.dtype == torch.float32:
        return MALA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("MALA tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("MALA tensors must be contiguous")


def _expect(t, name, shape, dtype):
    """The library sees raw pointers: every extent it derives from the sizes
    passed must match the tensor actually behind the pointer."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _expect_qkv(q, k, v, nq_dims=4):
    """q [B,H,L,d] (or [B,H,d] for decode) and k, v [B,Hkv,Lk,d] of q's dtype;
    returns (B, H, Hkv, Lk, d)."""
    if q.dim() != nq_dims or k.dim() != 4:
        raise ValueError(f"q must be {nq_dims}-D and k 4-D (got {q.dim()}-D and {k.dim()}-D)")
    _dt(q)
    B, H, d = q.shape[0], q.shape[1], q.shape[-1]
    Hkv, Lk = k.shape[1], k.shape[2]
    _expect(k, "k", (B, Hkv, Lk, d), q.dtype)
    _expect(v, "v", (B, Hkv, Lk, d), q.dtype)
    return B, H, Hkv, Lk, d


def _expect_stats(st, shapes):
    """Caller-supplied statistics buffers must be of the sizes and types the
    library writes (shapes: name -> shape; test_stat float32, the rest int32)."""
    if st is None:
        return
    for n, shape in shapes.items():
        if n in st and st[n] is not None:
            _expect(st[n], f"stats[{n!r}]", shape, torch.float32 if n == "test_stat" else torch.int32)
            _check_dev(st[n])
    if len(st.get("events", ())) > 4:
        raise ValueError("at most 4 events")


def _prefill_stat_shapes(B, H, nqb, ntiles):
    w = -(-ntiles // 32)
    return {"kept": (B, H, nqb), "legal": (B, H, nqb), "keep_bits": (B, H, nqb, w), "keep_bits_dkdv": (B, H, nqb, w),
            "test_stat": (B, H, nqb, ntiles)}


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def prefill_stats_buffers(B, H, L, tile, device, dkdv=False, test_stat=False, Lk=None):
    """Statistics buffers of a prefill call (Lk: key count when it differs
    from L, as in a chunk).  test_stat (bf16 only) starts as NaN: entries of
    tiles that are not tested stay NaN."""
    bq, bk = tile
    nqb, nt = -(-L // bq), -(-(L if Lk is None else Lk) // bk)
    words = -(-nt // 32)
    st = {"kept": torch.zeros(B, H, nqb, dtype=torch.int32, device=device),
          "legal": torch.zeros(B, H, nqb, dtype=torch.int32, device=device),
          "keep_bits": torch.zeros(B, H, nqb, words, dtype=torch.int32, device=device)}
    if dkdv:
        st["keep_bits_dkdv"] = torch.zeros(B, H, nqb, words, dtype=torch.int32, device=device)
    if test_stat:
        st["test_stat"] = torch.full((B, H, nqb, nt), float("nan"), dtype=torch.float32, device=device)
    return st


def _stats_struct(st):
    """Stats dict -> mala_stats.  Tensors under kept/legal/keep_bits/keep_bits_dkdv;
    optional "events": up to 4 torch.cuda.Event(enable_timing=True), recorded by
    the library around its kernels (see include/mala.h)."""
    if st is None:
        return None
    s = Stats(*(ctypes.c_void_p(st[n].data_ptr()) if n in st else None
                for n in ("kept", "legal", "keep_bits", "keep_bits_dkdv")))
    if st.get("test_stat") is not None:
        s.test_stat = ctypes.c_void_p(st["test_stat"].data_ptr())
    for i, ev in enumerate(st.get("events", ())):
        if ev is not None:
            if not ev.cuda_event:
                ev.record()  # torch creates the underlying event lazily
            s.events[i] = ev.cuda_event
    return ctypes.byref(s)


def fwd_into(q, k, v, o, lse, tau, tile=None, scale=0.0, stats=None, stream=None):
    """Queue mala_fwd writing into preallocated o [B,H,L,d] and lse [B,H,L] (fp32)."""
    B, H, Hkv, L, d = _expect_qkv(q, k, v)
    if q.shape[2] != L:
        raise ValueError(f"q has {q.shape[2]} rows but k, v have {L} (use fwd_chunk for a query chunk)")
    _expect(o, "o", q.shape, q.dtype)
    _expect(lse, "lse", (B, H, L), torch.float32)
    tile = tile or DEFAULT_TILE[q.dtype]
    _expect_stats(stats, _prefill_stat_shapes(B, H, -(-L // tile[0]), -(-L // tile[1])))
    _check_dev(q, k, v, o, lse)
    rc = _lib.load().mala_fwd(_ptr(q), _ptr(k), _ptr(v), B, H, k.shape[1], L, d, _dt(q), float(tau), Tile(*tile),
                              float(scale), _ptr(o), _ptr(lse), _stats_struct(stats), _stream(stream))
    _lib.check("mala_fwd", rc)


def fwd(q, k, v, tau, tile=None, scale=0.0, stats=False):
    """MALA forward.  Returns (o, lse) or (o, lse, stats dict)."""
    _check_dev(q, k, v)
    B, H, L, d = q.shape
    tile = tile or DEFAULT_TILE[q.dtype]
    o = torch.empty_like(q)
    lse = torch.empty(B, H, L, dtype=torch.float32, device=q.device)
    st = prefill_stats_buffers(B, H, L, tile, q.device, test_stat=q.dtype == torch.bfloat16) if stats else None
    fwd_into(q, k, v, o, lse, tau, tile, scale, st)
    return (o, lse, st) if stats else (o, lse)


def fwd_chunk_into(q, kc, vc, P, o, lse, tau, tile=None, scale=0.0, stats=None, stream=None):
    """Queue mala_fwd_chunk: q [B,H,Lq,d] at key positions P.., caches [B,Hkv,Lcap,d]
    holding keys 0 .. P+Lq-1; writes o [B,H,Lq,d] and lse [B,H,Lq]."""
    B, H, Hkv, Lcap, d = _expect_qkv(q, kc, vc)
    Lq = q.shape[2]
    _expect(o, "o", q.shape, q.dtype)
    _expect(lse, "lse", (B, H, Lq), torch.float32)
    tile = tile or DEFAULT_TILE[q.dtype]
    _expect_stats(stats, _prefill_stat_shapes(B, H, -(-Lq // tile[0]), -(-(int(P) + Lq) // tile[1])))
    _check_dev(q, kc, vc, o, lse)
    rc = _lib.load().mala_fwd_chunk(_ptr(q), _ptr(kc), _ptr(vc), B, H, Hkv, Lq, int(P), Lcap, d, _dt(q), float(tau),
                                    Tile(*tile), float(scale), _ptr(o), _ptr(lse), _stats_struct(stats),
                                    _stream(stream))
    _lib.check("mala_fwd_chunk", rc)


def fwd_chunk(q, kc, vc, P, tau, tile=None, scale=0.0, stats=False):
    """Chunked-prefill MALA forward against a K/V cache.  Returns (o, lse[, stats])."""
    _check_dev(q, kc, vc)
    B, H, Lq, d = q.shape
    tile = tile or DEFAULT_TILE[q.dtype]
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Lq, dtype=torch.float32, device=q.device)
    st = prefill_stats_buffers(B, H, Lq, tile, q.device, test_stat=True, Lk=int(P) + Lq) if stats else None
    fwd_chunk_into(q, kc, vc, P, o, lse, tau, tile, scale, st)
    return (o, lse, st) if stats else (o, lse)


def bwd_workspace(q, tile=None):
    B, H, L, d = q.shape
    tile = tile or DEFAULT_TILE[q.dtype]
    n = _lib.load().mala_bwd_workspace_size(B, H, L, d, _dt(q), Tile(*tile))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws, tile=None, scale=0.0, stats=None, stream=None):
    """Queue mala_bwd writing into preallocated dq (like q) and dk, dv (like k);
    ws from bwd_workspace."""
    B, H, Hkv, L, d = _expect_qkv(q, k, v)
    if q.shape[2] != L:
        raise ValueError(f"q has {q.shape[2]} rows but k, v have {L}")
    for t, n in ((o, "o"), (do, "do"), (dq, "dq")):
        _expect(t, n, q.shape, q.dtype)
    for t, n in ((dk, "dk"), (dv, "dv")):
        _expect(t, n, k.shape, q.dtype)
    _expect(lse, "lse", (B, H, L), torch.float32)
    if ws is None or ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError("ws must be a 1-D uint8 workspace (see bwd_workspace)")
    tile = tile or DEFAULT_TILE[q.dtype]
    _expect_stats(stats, _prefill_stat_shapes(B, H, -(-L // tile[0]), -(-L // tile[1])))
    _check_dev(q, k, v, o, lse, do, dq, dk, dv, ws)
    rc = _lib.load().mala_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), B, H, k.shape[1], L, d,
                              _dt(q), float(tau), Tile(*tile), float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                              _stats_struct(stats), _ptr(ws), ws.numel(), _stream(stream))
    _lib.check("mala_bwd", rc)


def bwd(q, k, v, o, lse, do, tau, tile=None, scale=0.0, stats=False):
    """MALA backward against forward state (o, lse).  Returns (dq, dk, dv[, stats])."""
    _check_dev(q, k, v, o, lse, do)
    B, H, L, d = q.shape
    tile = tile or DEFAULT_TILE[q.dtype]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = bwd_workspace(q, tile)
    st = prefill_stats_buffers(B, H, L, tile, q.device, dkdv=True, test_stat=q.dtype == torch.bfloat16) if stats else None
    bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws, tile, scale, st)
    return (dq, dk, dv, st) if stats else (dq, dk, dv)


class _MalaAttention(torch.autograd.Function):
    """Autograd binding: forward runs mala_fwd and keeps (o, lse) as the
    attention state; backward runs mala_bwd against it."""

    @staticmethod
    def forward(ctx, q, k, v, tau, tile, scale):
        o, lse = fwd(q, k, v, tau, tile, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.tau, ctx.tile, ctx.scale = tau, tile, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), ctx.tau, ctx.tile, ctx.scale)
        return dq, dk, dv, None, None, None


def mala_attention(q, k, v, tau=1.0, tile=None, scale=0.0):
    """Causal MALA attention with autograd, as a drop-in for a fused causal
    attention call.  q: [B, H, L, d]; k, v: [B, Hkv, L, d] with H % Hkv == 0
    (grouped-query attention when Hkv < H); bf16 with d = 128, or fp32 with
    d = 64 and H == Hkv.  Returns o: [B, H, L, d]."""
    return _MalaAttention.apply(q.contiguous(), k.contiguous(), v.contiguous(), float(tau), tile, float(scale))


def decode_stats_buffers(B, Hkv, Lk, split_keys, bk, device, vote_groups=1, test_stat=False):
    """Decode statistics for B sequences, Hkv KV heads and vote_groups vote
    groups per KV head (G / rows_per_vote; 1 when the whole group votes);
    test_stat starts as NaN."""
    nsplit = -(-Lk // split_keys)
    tps = split_keys // bk
    words = -(-tps // 32)
    V = Hkv * vote_groups
    st = {"kept": torch.zeros(B, V, nsplit, dtype=torch.int32, device=device),
          "legal": torch.zeros(B, V, nsplit, dtype=torch.int32, device=device),
          "keep_bits": torch.zeros(B, V, nsplit, words, dtype=torch.int32, device=device)}
    if test_stat:
        st["test_stat"] = torch.full((B, V, nsplit, tps), float("nan"), dtype=torch.float32, device=device)
    return st


def _vote_groups(Hq, Hkv, rows_per_vote):
    """Vote groups per KV head, or None when rows_per_vote does not divide
    G (the library rejects the call)."""
    G = Hq // Hkv
    R = int(rows_per_vote) or G
    return G // R if R > 0 and G % R == 0 else None


def decode_workspace(B, Hq, Hkv, Lk, d, split_keys, device):
    n = _lib.load().mala_decode_workspace_size(B, Hq, Hkv, Lk, d, split_keys)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def decode_into(q, kc, vc, Lk, o, lse, tau, ws, split_keys=4096, bk=64, scale=0.0, stats=None, stream=None,
                seeded=False, rows_per_vote=0):
    """Queue mala_decode (or mala_decode_seeded): q [B,Hq,d], caches
    [B,Hkv,Lcap,d] with Lk valid rows; writes o (like q) and lse [B,Hq] (or
    None); ws from decode_workspace.  rows_per_vote: query heads per vote
    (0: the whole KV group)."""
    B, Hq, Hkv, Lcap, d = _expect_qkv(q, kc, vc, nq_dims=3)
    _expect(o, "o", q.shape, q.dtype)
    if lse is not None:
        _expect(lse, "lse", (B, Hq), torch.float32)
    if ws is None or ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError("ws must be a 1-D uint8 workspace (see decode_workspace)")
    vg = _vote_groups(Hq, Hkv, rows_per_vote)
    if stats is not None and int(split_keys) > 0 and int(bk) > 0 and vg:  # (bad sizes: the library rejects them)
        nsplit, w = -(-int(Lk) // int(split_keys)), -(-(int(split_keys) // int(bk)) // 32)
        V = Hkv * vg
        _expect_stats(stats, {"kept": (B, V, nsplit), "legal": (B, V, nsplit), "keep_bits": (B, V, nsplit, w),
                              "test_stat": (B, V, nsplit, int(split_keys) // int(bk))})
    _check_dev(q, kc, vc, o, ws, *([lse] if lse is not None else []))
    name = "mala_decode_seeded" if seeded else "mala_decode"
    rc = getattr(_lib.load(), name)(_ptr(q), _ptr(kc), _ptr(vc), B, Hq, Hkv, int(Lk), Lcap, d, _dt(q), float(tau),
                                    int(split_keys), int(bk), int(rows_per_vote), float(scale), _ptr(o), _ptr(lse),
                                    _stats_struct(stats), _ptr(ws), ws.numel(), _stream(stream))
    _lib.check(name, rc)


def decode(q, kc, vc, Lk, tau, split_keys=4096, bk=64, scale=0.0, stats=False, seeded=False, rows_per_vote=0):
    """Split-KV MALA decode.  q [B,Hq,d], caches [B,Hkv,Lcap,d].  Returns (o, lse[, stats]).
    seeded=True runs mala_decode_seeded (partitions counted back from the
    newest tile, the older ones tested against the newest one's state).
    rows_per_vote: query heads per vote (0: the whole KV group votes)."""
    _check_dev(q, kc, vc)
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    ws = decode_workspace(B, Hq, Hkv, Lk, d, split_keys, q.device)
    st = None
    if stats:
        st = decode_stats_buffers(B, Hkv, Lk, split_keys, bk, q.device, _vote_groups(Hq, Hkv, rows_per_vote) or 1,
                                  test_stat=True)
    decode_into(q, kc, vc, Lk, o, lse, tau, ws, split_keys, bk, scale, st, seeded=seeded,
                rows_per_vote=rows_per_vote)
    return (o, lse, st) if stats else (o, lse)


def decode_noalloc_into(q, kc, vc, Lk, o, lse, tau, split_keys=4096, bk=64, scale=0.0, stats=None, stream=None,
                        rows_per_vote=0):
    """Queue mala_decode_noalloc: mala_decode with the split partials in the
    library's static device scratch (no workspace, no device allocation by
    the library); writes o (like q) and lse [B,Hq] (or None).  Calls that
    overlap on one GPU share that scratch: keep them on one stream."""
    B, Hq, Hkv, Lcap, d = _expect_qkv(q, kc, vc, nq_dims=3)
    _expect(o, "o", q.shape, q.dtype)
    if lse is not None:
        _expect(lse, "lse", (B, Hq), torch.float32)
    vg = _vote_groups(Hq, Hkv, rows_per_vote)
    if stats is not None and int(split_keys) > 0 and int(bk) > 0 and vg:
        nsplit, w = -(-int(Lk) // int(split_keys)), -(-(int(split_keys) // int(bk)) // 32)
        V = Hkv * vg
        _expect_stats(stats, {"kept": (B, V, nsplit), "legal": (B, V, nsplit), "keep_bits": (B, V, nsplit, w),
                              "test_stat": (B, V, nsplit, int(split_keys) // int(bk))})
    _check_dev(q, kc, vc, o, *([lse] if lse is not None else []))
    rc = _lib.load().mala_decode_noalloc(_ptr(q), _ptr(kc), _ptr(vc), B, Hq, Hkv, int(Lk), Lcap, d, _dt(q),
                                         float(tau), int(split_keys), int(bk), int(rows_per_vote), float(scale),
                                         _ptr(o), _ptr(lse), _stats_struct(stats), _stream(stream))
    _lib.check("mala_decode_noalloc", rc)


def bits_to_keep(bits, ntiles):
    """Unpack int32 keep-bit words [..., words] to a uint8 array [..., ntiles] (numpy)."""
    import numpy as np
    b = bits.cpu().numpy().astype(np.uint32)
    idx = np.arange(ntiles)
    return ((b[..., idx // 32] >> (idx % 32).astype(np.uint32)) & 1).astype(np.uint8)


def default_scale(d):
    return 1.0 / math.sqrt(d)
