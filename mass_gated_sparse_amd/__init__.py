"""MassAlloc Attention (MALA) for AMD Instinct MI355X (gfx950).

The operator lives in libmala.so (hand-written HIP kernels behind the C ABI
of include/mala.h); this package only builds it and marshals arguments.
"""
from .build import build, lib_path  # noqa: F401
