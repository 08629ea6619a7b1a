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
