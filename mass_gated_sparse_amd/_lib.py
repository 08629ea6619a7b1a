"""ctypes binding of libmala.so (the C ABI declared in include/mala.h).

Argument marshalling only: every step of the operator runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library has not been built this module raises; there is no fallback path.
"""
import ctypes
import os

from .build import lib_path

MALA_BF16, MALA_F32 = 0, 1
_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported configuration", -3: "HIP runtime error"}


class MalaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({status}): {msg}")
        self.status = status


class Tile(ctypes.Structure):
    _fields_ = [("bq", ctypes.c_int), ("bk", ctypes.c_int)]


class Stats(ctypes.Structure):
    _fields_ = [("kept", ctypes.c_void_p), ("legal", ctypes.c_void_p), ("keep_bits", ctypes.c_void_p),
                ("keep_bits_dkdv", ctypes.c_void_p), ("events", ctypes.c_void_p * 4), ("test_stat", ctypes.c_void_p)]


EXPORTS = ("mala_fwd", "mala_fwd_chunk", "mala_bwd", "mala_bwd_workspace_size", "mala_decode", "mala_decode_seeded",
           "mala_decode_noalloc", "mala_decode_workspace_size", "mala_status_string", "mala_last_error",
           "mala_version")
# bytes of the static device scratch behind mala_decode_noalloc (MALA_DECODE_NOALLOC_SCRATCH_BYTES)
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

_LIB = None


def load(path=None):
    """Load libmala.so and declare every exported signature."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or lib_path()
    if not os.path.exists(p):
        raise RuntimeError(f"libmala.so not found at {p}: build it first (python -m mass_gated_sparse_amd.build "
                           "or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sp = ctypes.POINTER(Stats)
    lib.mala_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, i, f, Tile, f, vp, vp, sp, vp]
    lib.mala_fwd.restype = i
    lib.mala_fwd_chunk.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, f, Tile, f, vp, vp, sp, vp]
    lib.mala_fwd_chunk.restype = i
    lib.mala_bwd_workspace_size.argtypes = [i, i, i, i, i, Tile]
    lib.mala_bwd_workspace_size.restype = sz
    lib.mala_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, Tile, f, vp, vp, vp, sp, vp, sz, vp]
    lib.mala_bwd.restype = i
    lib.mala_decode_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.mala_decode_workspace_size.restype = sz
    lib.mala_decode.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i, f, vp, vp, sp, vp, sz, vp]
    lib.mala_decode.restype = i
    lib.mala_decode_seeded.argtypes = lib.mala_decode.argtypes
    lib.mala_decode_seeded.restype = i
    lib.mala_decode_noalloc.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i, f, vp, vp, sp, vp]
    lib.mala_decode_noalloc.restype = i
    lib.mala_status_string.argtypes = [i]
    lib.mala_status_string.restype = ctypes.c_char_p
    lib.mala_last_error.argtypes = []
    lib.mala_last_error.restype = ctypes.c_char_p
    lib.mala_version.argtypes = []
    lib.mala_version.restype = i
    if path is None:
        _LIB = lib
    return lib


def check(fn, status):
    if status != 0:
        raise MalaError(fn, status, load().mala_last_error().decode())
