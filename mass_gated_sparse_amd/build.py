"""Builds libmala.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["mala_api.hip", "mala_fwd.hip", "mala_bwd.hip", "mala_decode.hip", "mala_simple.hip"]
ARCH = "gfx950"
# -packed-fp32-ops: no packed fp32 VALU instructions are generated.
# -Werror=shadow-all: kernels are long lambdas over many locals; a name that
#   shadows one of them (a compile-time tag named like a kernel argument) is
#   an error, not a silent change of meaning.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Werror=shadow-all",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# -amdgpu-mfma-vgpr-form: MFMA results go to arch VGPRs first.  Kernels that
#   run two waves per SIMD (256 registers each) then avoid per-iteration
#   AGPR<->VGPR copies and scratch spills.  FILE_FLAGS replaces it for a
#   source that needs other code-generation flags (none at present).
MFMA_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
FILE_FLAGS = {}


def lib_path() -> str:
    return os.path.join(HERE, "libmala.so")


def ubench_path() -> str:
    return os.path.join(HERE, "libmala_ubench.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    return msg


def _hipcc(srcs, out, verbose, extra=()):
    """Compile every source to an object with its own flags, then link one
    shared library."""
    import shutil
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmpdir = tempfile.mkdtemp(prefix="mala_build_")
    try:
        def obj(src):
            o = os.path.join(tmpdir, os.path.basename(src) + ".o")
            flags = FILE_FLAGS.get(os.path.basename(src), MFMA_VGPR_FORM)
            return o, _run([hipcc, *HIPCC_FLAGS, *flags, *extra, "-c", src, "-o", o])
        with ThreadPoolExecutor(min(8, len(srcs))) as ex:
            res = list(ex.map(obj, srcs))
        tmp = out + ".tmp"
        msgs = [m for _, m in res] + [_run([hipcc, *HIPCC_FLAGS, "-shared", *[o for o, _ in res], "-o", tmp])]
        if verbose and any(m.strip() for m in msgs):
            print("\n".join(m for m in msgs if m.strip()))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


def build(verbose: bool = False) -> str:
    """Compile libmala.so (the operator) and libmala_ubench.so (ceiling
    microbenchmarks used by bench.py --micro) side by side."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(2) as ex:
        f1 = ex.submit(_hipcc, [os.path.join(CSRC, s) for s in SOURCES], lib_path(), verbose)
        f2 = ex.submit(_hipcc, [os.path.join(CSRC, "mala_ubench.hip")], ubench_path(), verbose)
        f2.result()
        return f1.result()


if __name__ == "__main__":
    print(build(verbose=True))
