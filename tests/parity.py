"""Helpers shared by the GPU parity tests: comparison rules against the oracle.

Rules (MALA digest, forward and backward paragraphs; tolerances as stated for
this operator): decisions are compared tile by tile and must be identical,
except that forward/decode tiles whose oracle statistic T lies within 1e-4 of
the threshold (|T - 1| <= 1e-4) are listed and excluded -- there either
decision is correct, and the oracle is run in replay mode so it follows the
GPU through them.  Outputs are compared by relative L2 over the tensor.
"""
import numpy as np

BAND = 1e-4
TOL_O = 5e-3
TOL_GRAD = 1e-2


def rel_l2(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return float(np.linalg.norm((x - y).ravel()) / max(np.linalg.norm(y.ravel()), 1e-300))


def legal_mask(L, bq, bk):
    nqb, nt = -(-L // bq), -(-L // bk)
    jmax = (np.minimum(np.arange(nqb) * bq + bq, L) - 1) // bk
    return np.arange(nt)[None, :] <= jmax[:, None]


def chunk_legal_mask(Lq, P, bq, bk):
    """Legal tiles of a query chunk at key offset P: block b sees keys up to
    P + min(b*bq + bq, Lq) - 1."""
    nqb, nt = -(-Lq // bq), -(-(P + Lq) // bk)
    jmax = (P + np.minimum(np.arange(nqb) * bq + bq, Lq) - 1) // bk
    return np.arange(nt)[None, :] <= jmax[:, None]


def decision_report(gpu_keep, ora_keep, ora_T, legal, band=BAND):
    """Returns (n_bad, n_near, near_list): mismatches outside the band, tiles in the band."""
    legal = np.broadcast_to(legal, gpu_keep.shape)
    near = legal & np.isfinite(ora_T) & (np.abs(ora_T - 1.0) <= band)
    bad = legal & (gpu_keep != ora_keep) & ~near
    near_list = [tuple(int(x) for x in idx) + (float(ora_T[idx]), int(gpu_keep[idx]), int(ora_keep[idx]))
                 for idx in zip(*np.nonzero(near))]
    return int(bad.sum()), int(near.sum()), near_list


def bf16_to_f64(t):
    """fp64 numpy values of a torch bf16/fp32 tensor."""
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


# log2 units: fp32 scores and running sums against fp64.  Measured worst
# differences are 1.4e-5 (prefill, L <= 4096) and 5e-6 (decode); 1e-4 stays
# below the 1.44e-4 that the |T - 1| <= 1e-4 decision band spans in log2 T,
# so a statistic within it cannot flip a decision outside the band.
TOL_TSTAT = 1e-4


def tstat_report(gpu_ts, ora_T, legal, tau):
    """The GPU's per-tile statistic (log2 T) against the oracle's T on every
    legal tile: returns (worst |difference| over tiles where both are finite,
    number of tiles where they disagree otherwise).  At tau = 0 the GPU writes
    NaN (no test is run)."""
    g = np.asarray(gpu_ts, dtype=np.float64)
    legal = np.broadcast_to(legal, g.shape)
    if tau == 0.0:
        return 0.0, int((legal & ~np.isnan(g)).sum())
    with np.errstate(divide="ignore"):
        o = np.log2(np.asarray(ora_T, dtype=np.float64))
    fin = legal & np.isfinite(g) & np.isfinite(o)
    worst = float(np.abs(g[fin] - o[fin]).max()) if fin.any() else 0.0
    other = legal & ~fin
    bad = int((other & ~(np.isinf(g) & np.isinf(o) & (np.sign(g) == np.sign(o)))).sum())
    return worst, bad

