"""mala_decode_noalloc against mala_decode on the GPU, through the C ABI.

The entry point for callers that cannot allocate keeps the split partials in
the library's static device scratch; it must give exactly what mala_decode
gives with a caller's workspace (the same kernels), call after call, with the
scratch holding the previous call's contents: first at the full 128K decode
shape (8.8 MB of partials), then at a smaller shape, then the first shape
again with one vote per query head.
"""
import numpy as np
import pytest

from synth import WORKLOADS, decode_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mass_gated_sparse_amd import ops as _ops
    return _ops


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _case(Lk, batches, Lcap=None):
    w = WORKLOADS["decode128k"]
    x = decode_inputs(w, Lk=Lk, Lcap=Lcap, batches=batches, threads=16)
    x = {n: np.ascontiguousarray(a[list(batches)]) for n, a in x.items()}
    return w, tuple(_dev(x[n]) for n in ("q", "k", "v"))


def _both(ops, q, kc, vc, Lk, tau, split, rpv=0):
    """(o, lse, stats) of mala_decode with a workspace and of
    mala_decode_noalloc, on the same stream, one after the other."""
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    vg = G // (rpv or G)
    out = []
    for noalloc in (False, True):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
        st = ops.decode_stats_buffers(B, Hkv, Lk, split, 64, q.device, vote_groups=vg)
        if noalloc:
            ops.decode_noalloc_into(q, kc, vc, Lk, o, lse, tau, split_keys=split, stats=st, rows_per_vote=rpv)
        else:
            ws = ops.decode_workspace(B, Hq, Hkv, Lk, d, split, q.device)
            ops.decode_into(q, kc, vc, Lk, o, lse, tau, ws, split_keys=split, stats=st, rows_per_vote=rpv)
        out.append((o, lse, st))
    torch.cuda.synchronize()
    return out


def _same(a, b):
    (o1, l1, s1), (o2, l2, s2) = a, b
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for n in ("kept", "legal", "keep_bits"):
        assert torch.equal(s1[n], s2[n]), n


def test_noalloc_decode_equals_workspace_decode(ops):
    w = WORKLOADS["decode128k"]
    print("case: full decode shape (16 x 32 heads, 131073 keys), tau=1", flush=True)
    _, (q, kc, vc) = _case(w.L, tuple(range(w.B)))
    _same(*_both(ops, q, kc, vc, w.L, 1.0, w.split_keys))
    print("case: 3 sequences, 5000 keys of a 5003-row cache, split 1024, tau=1", flush=True)
    _, (q2, kc2, vc2) = _case(5000, (0, 1, 2), Lcap=5003)
    _same(*_both(ops, q2, kc2, vc2, 5000, 1.0, 1024))
    print("case: full decode shape again, one vote per query head, tau=0 and tau=1", flush=True)
    _same(*_both(ops, q, kc, vc, w.L, 0.0, w.split_keys))
    _same(*_both(ops, q, kc, vc, w.L, 1.0, w.split_keys, rpv=1))


def test_noalloc_decode_rejects_beyond_scratch(ops):
    """A call needing more partials than the scratch holds fails before
    anything is queued."""
    from mass_gated_sparse_amd._lib import DECODE_NOALLOC_SCRATCH_BYTES, MalaError
    q = torch.zeros(64, 64, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(64, 8, 4096, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    nsplit = 4096 // 64
    assert 64 * 64 * nsplit * 130 * 4 > DECODE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(MalaError) as e:
        ops.decode_noalloc_into(q, kc, kc, 4096, o, None, 1.0, split_keys=64)
    assert e.value.status == -2 and "static scratch" in str(e.value)
