"""Host-side checks of the C ABI in include/mala.h (no GPU needed).

The library must load, export every function the header declares, and reject
bad arguments on the host before any HIP call: every call below fails
validation, so the dummy pointers handed in are never dereferenced and no
kernel is launched.
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mala.h")

OK, INVALID, UNSUPPORTED, HIPERR = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(mala_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from mass_gated_sparse_amd import _lib
    from mass_gated_sparse_amd.build import lib_path
    if not os.path.exists(lib_path()):
        pytest.fail("libmala.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_the_documented_entry_points():
    fns = declared_functions()
    for name in ("mala_fwd", "mala_fwd_chunk", "mala_bwd", "mala_decode", "mala_decode_seeded", "mala_decode_noalloc",
                 "mala_bwd_workspace_size", "mala_decode_workspace_size", "mala_status_string", "mala_last_error",
                 "mala_version"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    from mass_gated_sparse_amd import _lib
    raw = ctypes.CDLL(lib._name)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, missing
    assert sorted(_lib.EXPORTS) == declared_functions()


def test_version_and_status_strings(lib):
    assert lib.mala_version() == 103
    assert lib.mala_status_string(OK) == b"ok"
    assert lib.mala_status_string(INVALID) == b"invalid argument"
    assert lib.mala_status_string(UNSUPPORTED) == b"unsupported configuration"
    assert lib.mala_status_string(HIPERR) == b"HIP runtime error"
    assert lib.mala_status_string(7) == b"unknown status"


def test_workspace_sizes(lib):
    from mass_gated_sparse_amd._lib import MALA_BF16, Tile
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for B, H, L in [(1, 4, 131072), (2, 3, 1000), (1, 1, 1)]:
        words = -(-(-(-L // 64)) // 32)
        assert lib.mala_bwd_workspace_size(B, H, L, 128, MALA_BF16, Tile(128, 64)) == (
            3 * a256(B * H * L * 4) + a256(B * H * (-(-L // 128)) * words * 4))
    assert lib.mala_bwd_workspace_size(0, 4, 10, 128, MALA_BF16, Tile(128, 64)) == 0
    for B, Hq, Hkv, Lk, d, split in [(16, 32, 8, 131073, 128, 4096), (1, 4, 1, 2500, 128, 1024), (3, 8, 2, 64, 128, 64)]:
        nsplit = math.ceil(Lk / split)
        tiles = a256(B * Hq * (split // 64) * (d + 2) * 4) if nsplit > 1 and split // 64 <= 256 else 0
        assert lib.mala_decode_workspace_size(B, Hq, Hkv, Lk, d, split) == a256(B * Hq * nsplit * (d + 2) * 4) + tiles
    assert lib.mala_decode_workspace_size(1, 4, 1, 0, 128, 4096) == 0


P = ctypes.c_void_p(1 << 20)  # dummy, never dereferenced (validation fails first)
ALIGNED_WS = ctypes.c_void_p(1 << 20)
MISALIGNED_WS = ctypes.c_void_p((1 << 20) + 16)


def fwd(lib, q=P, B=1, H=2, Hkv=2, L=256, d=128, dt=0, tau=1.0, tile=(128, 64), o=P, lse=P):
    from mass_gated_sparse_amd._lib import Tile
    return lib.mala_fwd(q, P, P, B, H, Hkv, L, d, dt, tau, Tile(*tile), 0.0, o, lse, None, None)


@pytest.mark.parametrize("kw,status,msg", [
    ({"q": None}, INVALID, "null input"),
    ({"o": None}, INVALID, "null output"),
    ({"L": 0}, INVALID, "positive"),
    ({"B": -1}, INVALID, "positive"),
    ({"tau": -0.5}, INVALID, "tau"),
    ({"tau": float("nan")}, INVALID, "tau"),
    ({"dt": 5}, INVALID, "dtype"),
    ({"tile": (0, 64)}, INVALID, "tile"),
    ({"H": 4, "Hkv": 3}, INVALID, "multiple"),
    ({"H": 4, "Hkv": 2, "dt": 1, "d": 64, "tile": (64, 64)}, UNSUPPORTED, "grouped"),  # f32 path: H == Hkv only
    ({"d": 64}, UNSUPPORTED, "instantiation"),
    ({"tile": (64, 64)}, UNSUPPORTED, "instantiation"),
    ({"dt": 1}, UNSUPPORTED, "instantiation"),  # f32 path is d=64 only
    ({"B": 1 << 12, "H": 1 << 12, "Hkv": 1 << 12, "L": 1 << 10}, UNSUPPORTED, "too large"),
    ({"L": 1 << 24}, UNSUPPORTED, "too long"),
])
def test_fwd_rejects(lib, kw, status, msg):
    assert fwd(lib, **kw) == status
    assert msg in lib.mala_last_error().decode()


def fwd_chunk(lib, q=P, B=1, H=4, Hkv=2, Lq=256, Poff=1000, Lcap=2048, d=128, dt=0, tau=1.0, tile=(128, 64),
              o=P, lse=P):
    from mass_gated_sparse_amd._lib import Tile
    return lib.mala_fwd_chunk(q, P, P, B, H, Hkv, Lq, Poff, Lcap, d, dt, tau, Tile(*tile), 0.0, o, lse, None, None)


@pytest.mark.parametrize("kw,status,msg", [
    ({"q": None}, INVALID, "null input"),
    ({"lse": None}, INVALID, "null output"),
    ({"Poff": -1}, INVALID, "offset"),
    ({"Lcap": 1255}, INVALID, "exceeds Lcap"),
    ({"Lq": 0}, INVALID, "positive"),
    ({"tau": float("nan")}, INVALID, "tau"),
    ({"H": 4, "Hkv": 3}, INVALID, "multiple"),
    ({"dt": 1, "d": 64, "tile": (64, 64), "H": 2, "Hkv": 2}, UNSUPPORTED, "bf16"),
    ({"d": 64}, UNSUPPORTED, "instantiation"),
    ({"Lcap": 1 << 24}, UNSUPPORTED, "too long"),
])
def test_fwd_chunk_rejects(lib, kw, status, msg):
    assert fwd_chunk(lib, **kw) == status
    assert msg in lib.mala_last_error().decode()


def test_test_stat_layout_and_fp32_rejection(lib):
    """mala_stats ends with the test_stat pointer (after the four events);
    the fp32 path does not write it and says so before queuing anything."""
    from mass_gated_sparse_amd._lib import Stats, Tile
    assert Stats.test_stat.offset == 8 * 8 and ctypes.sizeof(Stats) == 9 * 8
    st = Stats()
    st.test_stat = P
    rc = lib.mala_fwd(P, P, P, 1, 2, 2, 256, 64, 1, 1.0, Tile(64, 64), 0.0, P, P, ctypes.byref(st), None)
    assert rc == UNSUPPORTED and "test_stat" in lib.mala_last_error().decode()
    rc = lib.mala_bwd(P, P, P, P, P, P, 1, 2, 2, 256, 64, 1, 1.0, Tile(64, 64), 0.0, P, P, P, ctypes.byref(st),
                      ALIGNED_WS, 1 << 30, None)
    assert rc == UNSUPPORTED and "test_stat" in lib.mala_last_error().decode()


def bwd(lib, ws=ALIGNED_WS, ws_bytes=1 << 30, dq=P, dout=P, tau=1.0, d=128):
    from mass_gated_sparse_amd._lib import Tile
    return lib.mala_bwd(P, P, P, P, P, dout, 1, 2, 2, 256, d, 0, tau, Tile(128, 64), 0.0, dq, P, P, None,
                        ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    ({"dout": None}, INVALID, "dout"),
    ({"dq": None}, INVALID, "gradient"),
    ({"ws": None}, INVALID, "workspace too small"),
    ({"ws_bytes": 100}, INVALID, "workspace too small"),
    ({"ws": MISALIGNED_WS}, INVALID, "aligned"),
    ({"tau": -1.0}, INVALID, "tau"),
    ({"d": 96}, UNSUPPORTED, "instantiation"),
])
def test_bwd_rejects(lib, kw, status, msg):
    assert bwd(lib, **kw) == status
    assert msg in lib.mala_last_error().decode()


def dec(lib, q=P, B=2, Hq=8, Hkv=2, Lk=5000, Lcap=8192, d=128, dt=0, tau=1.0, split=4096, bk=64, rpv=0,
        ws=ALIGNED_WS, ws_bytes=1 << 30, fn="mala_decode"):
    return getattr(lib, fn)(q, P, P, B, Hq, Hkv, Lk, Lcap, d, dt, tau, split, bk, rpv, 0.0, P, P, None, ws,
                            ws_bytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    ({"q": None}, INVALID, "null"),
    ({"Lk": 0}, INVALID, "positive"),
    ({"Lcap": 4000}, INVALID, "Lcap"),
    ({"tau": -2.0}, INVALID, "tau"),
    ({"Hq": 6, "Hkv": 4}, INVALID, "multiple"),
    ({"dt": 3}, INVALID, "dtype"),
    ({"dt": 1}, UNSUPPORTED, "instantiation"),
    ({"d": 64}, UNSUPPORTED, "instantiation"),
    ({"bk": 32}, UNSUPPORTED, "instantiation"),
    ({"Hq": 32, "Hkv": 2}, UNSUPPORTED, "instantiation"),  # group of 16 > 8
    ({"Hq": 24, "Hkv": 8}, UNSUPPORTED, "instantiation"),  # group of 3: no kernel for it
    ({"Hq": 12, "Hkv": 2}, UNSUPPORTED, "instantiation"),  # group of 6
    ({"Hq": 7, "Hkv": 1}, UNSUPPORTED, "instantiation"),   # group of 7
    ({"split": 4000}, UNSUPPORTED, "instantiation"),      # not a multiple of 64
    ({"ws_bytes": 64}, INVALID, "workspace too small"),
    ({"ws": MISALIGNED_WS}, INVALID, "aligned"),
    ({"rpv": 3}, INVALID, "rows_per_vote"),                # does not divide G = 4
    ({"rpv": -1}, INVALID, "rows_per_vote"),
    ({"rpv": 8}, INVALID, "rows_per_vote"),
])
@pytest.mark.parametrize("fn", ["mala_decode", "mala_decode_seeded"])
def test_decode_rejects(lib, kw, status, msg, fn):
    assert dec(lib, fn=fn, **kw) == status
    assert msg in lib.mala_last_error().decode()


def test_error_is_cleared_by_next_call(lib):
    assert fwd(lib, q=None) == INVALID
    assert lib.mala_last_error() != b""
    assert dec(lib, Lk=0) == INVALID
    assert b"positive" in lib.mala_last_error()


def test_python_wrappers_reject_host_tensors():
    import torch
    from mass_gated_sparse_amd import ops
    x = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        ops.fwd(x, x, x, 1.0)
    with pytest.raises(ValueError, match="GPU"):
        ops.decode(x[0], x, x, 128, 1.0)


def test_python_error_carries_library_message(lib):
    from mass_gated_sparse_amd import _lib
    assert fwd(lib, tau=-1.0) == INVALID
    with pytest.raises(_lib.MalaError, match="tau must be >= 0"):
        _lib.check("mala_fwd", INVALID)


def test_python_wrappers_check_shapes_before_the_device():
    """The C ABI sees raw pointers, so the binding checks every tensor's
    shape and dtype against the sizes it passes (on host tensors these checks
    fail before anything touches a device)."""
    import torch
    from mass_gated_sparse_amd import ops
    bf = torch.bfloat16

    def z(*s, dt=bf):
        return torch.zeros(*s, dtype=dt)
    q, k = z(1, 4, 256, 128), z(1, 2, 256, 128)
    o, lse = z(1, 4, 256, 128), z(1, 4, 256, dt=torch.float32)
    cases = [
        (lambda: ops.fwd_into(q, z(1, 2, 200, 128), k, o, lse, 1.0), "shape"),        # k rows differ
        (lambda: ops.fwd_into(q, k, z(1, 2, 256, 128, dt=torch.float32), o, lse, 1.0), "dtype"),
        (lambda: ops.fwd_into(q, k, k, o, z(1, 4, 255, dt=torch.float32), 1.0), "lse"),
        (lambda: ops.fwd_into(z(1, 4, 300, 128), k, k, z(1, 4, 300, 128), z(1, 4, 300, dt=torch.float32), 1.0),
         "rows"),
        (lambda: ops.fwd_into(q, k, k, o, lse, 1.0, stats={"kept": z(1, 4, 1, dt=torch.int32)}), "kept"),
        (lambda: ops.fwd_chunk_into(q, k, z(1, 2, 300, 128), 0, o, lse, 1.0), "shape"),
        (lambda: ops.bwd_into(q, k, k, o, lse, o, o, z(1, 4, 256, 128), k, 1.0, z(1024, dt=torch.uint8)), "dk"),
        (lambda: ops.bwd_into(q, k, k, o, lse, o, o, k, k, 1.0, z(16, dt=torch.float32)), "workspace"),
        (lambda: ops.decode_into(z(2, 8, 128), z(2, 2, 512, 128), z(2, 2, 500, 128), 500, z(2, 8, 128),
                                 z(2, 8, dt=torch.float32), 1.0, z(4096, dt=torch.uint8)), "shape"),
        (lambda: ops.decode_into(z(2, 8, 128), z(2, 2, 512, 128), z(2, 2, 512, 128), 500, z(2, 8, 128),
                                 z(2, 8, dt=torch.float32), 1.0, z(4096, dt=torch.uint8), split_keys=128,
                                 stats={"keep_bits": z(2, 2, 1, 1, dt=torch.int32)}), "keep_bits"),
        (lambda: ops.fwd_into(q, k, k, o, lse, 1.0, stats={"test_stat": z(1, 4, 2, 4)}), "test_stat"),  # bf16, not f32
        # one vote per query head: statistics are per head (8), not per KV head (2)
        (lambda: ops.decode_into(z(2, 8, 128), z(2, 2, 512, 128), z(2, 2, 512, 128), 500, z(2, 8, 128),
                                 z(2, 8, dt=torch.float32), 1.0, z(4096, dt=torch.uint8), split_keys=128,
                                 rows_per_vote=1, stats={"kept": z(2, 2, 4, dt=torch.int32)}), "kept"),
    ]
    for fn, msg in cases:
        with pytest.raises(ValueError, match=msg):
            fn()


def dec_noalloc(lib, q=P, B=2, Hq=8, Hkv=2, Lk=5000, Lcap=8192, d=128, dt=0, tau=1.0, split=4096, bk=64, rpv=0):
    return lib.mala_decode_noalloc(q, P, P, B, Hq, Hkv, Lk, Lcap, d, dt, tau, split, bk, rpv, 0.0, P, P, None, None)


@pytest.mark.parametrize("kw,status,msg", [
    ({"q": None}, INVALID, "null"),
    ({"Lcap": 4000}, INVALID, "Lcap"),
    ({"tau": float("nan")}, INVALID, "tau"),
    ({"Hq": 24, "Hkv": 8}, UNSUPPORTED, "instantiation"),
    ({"rpv": 3}, INVALID, "rows_per_vote"),
    # 64 x 64 x 33 x 130 x 4 bytes of partials: beyond the 16 MiB scratch
    ({"B": 64, "Hq": 64, "Hkv": 8, "Lk": 131073, "Lcap": 131073}, UNSUPPORTED, "static scratch"),
    ({"B": 1, "Hq": 8, "Hkv": 8, "Lk": 1 << 24, "Lcap": 1 << 24, "split": 64}, UNSUPPORTED, "static scratch"),
])
def test_decode_noalloc_rejects(lib, kw, status, msg):
    """mala_decode_noalloc checks every argument, and that the split partials
    fit its static scratch, before it touches the device."""
    assert dec_noalloc(lib, **kw) == status
    assert msg in lib.mala_last_error().decode()


def test_decode_noalloc_limit_matches_header():
    from mass_gated_sparse_amd import _lib
    text = open(HEADER).read()
    m = re.search(r"#define MALA_DECODE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.DECODE_NOALLOC_SCRATCH_BYTES
