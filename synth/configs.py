"""Named workloads for MassAlloc Attention (MALA).

Each workload is a fixed shape plus the seed of its synthetic inputs.  The
shapes follow the settings the MassAlloc Attention digest (agihunt.info,
"MassAlloc Attention: Let Attention Allocate Its Own Compute") reports on:
its operator-benchmark paragraph (128K tokens under 8-way head tensor
parallelism, so one GPU holds 4 of 32 heads), its matched-work paragraph (8K)
and its fidelity paragraph (1K to 32K).  The pages fix no tile size; the
tile shapes here are this implementation's choice.
"""
from dataclasses import dataclass

SEED_BASE = 20260926


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # seed offset: seed = SEED_BASE + index
    kind: str             # "prefill" (fwd+bwd) or "decode"
    B: int
    H: int                # query heads
    Hkv: int              # key/value heads
    L: int                # prefill: sequence length; decode: valid keys Lk (incl. new token)
    d: int
    dtype: str            # "bf16" or "f32"
    bq: int               # query rows per vote block (prefill); decode: rows of one GQA group
    bk: int               # keys per tile
    taus: tuple = (1.0,)
    sharp_lo: float = 0.5  # per-head sharpness multiplier c_h ~ U[lo, hi]
    sharp_hi: float = 2.0
    split_keys: int = 0   # decode only: keys per split-KV partition
    note: str = ""

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def group(self) -> int:
        return self.H // self.Hkv


TINY = Workload("tiny", 0, "prefill", B=1, H=2, Hkv=2, L=1024, d=64, dtype="f32",
                bq=64, bk=64, taus=(1.0, 0.0), sharp_lo=1.0, sharp_hi=1.0,
                note="tiny causal fwd+bwd, fp32, 64x64 tiles")
MW8K = Workload("mw8k", 1, "prefill", B=1, H=16, Hkv=16, L=8192, d=128, dtype="bf16",
                bq=128, bk=64, taus=(1.0,),
                note="8K matched-work study shape, bf16, 128x64 tiles")
SWEEP32K = Workload("sweep32k", 2, "prefill", B=1, H=8, Hkv=8, L=32768, d=128, dtype="bf16",
                    bq=128, bk=64, taus=(0.0, 0.5, 1.0, 2.0),
                    note="32K tau sweep; planted, planted with c=1 on every head, and diffuse families")
TRAIN128K = Workload("train128k", 3, "prefill", B=1, H=4, Hkv=4, L=131072, d=128, dtype="bf16",
                     bq=128, bk=64, taus=(1.0, 0.0),
                     note="128K training shape: one GPU's 4-head share of a 32-head layer")
DECODE128K = Workload("decode128k", 4, "decode", B=16, H=32, Hkv=8, L=131073, d=128, dtype="bf16",
                      bq=4, bk=64, taus=(1.0, 0.0), split_keys=4096,
                      note="128K decode: 16 sequences, GQA 32/8, one new token, split-KV 4096")

GQA8K = Workload("gqa8k", 5, "prefill", B=1, H=8, Hkv=2, L=8192, d=128, dtype="bf16",
                 bq=128, bk=64, taus=(1.0, 0.0),
                 note="grouped-query prefill: 8 query heads over 2 K/V heads (4 per group), bf16, 128x64 tiles")

WORKLOADS = {w.name: w for w in (TINY, MW8K, SWEEP32K, TRAIN128K, DECODE128K, GQA8K)}
