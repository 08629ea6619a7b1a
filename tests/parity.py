"""Helpers shared by the GPU parity tests: comparison rules against the oracle.

Rules (MassAlloc Attention digest at agihunt.info, forward and backward
paragraphs; tolerances as stated for this operator):

- Forward and decode decisions are compared tile by tile and must be
  identical, except on tiles whose oracle statistic T lies within 1e-4 of the
  threshold (|T - 1| <= 1e-4).  There either decision is correct; the oracle
  runs in replay mode so it follows the GPU through them, and every such tile
  is listed (printed) by the test.
- Backward decisions are compared without replay: every legal tile must take
  the oracle's decision, and the per-block kept counts must equal the
  oracle's sums.  Tiles in the band are printed as a diagnostic only.
- Outputs: relative L2 over the tensor (O <= 5e-3, dQ/dK/dV <= 1e-2), and
  every row within its rounding bound (see row_bounds).
"""
import math

import numpy as np

BAND = 1e-4
TOL_O = 5e-3
TOL_GRAD = 1e-2


def rel_l2(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return float(np.linalg.norm((x - y).ravel()) / max(np.linalg.norm(y.ravel()), 1e-300))


# Per-row bounds, from the rounding the kernels do (probabilistic rounding-error
# analysis: independent rounding errors add in quadrature).  With u = 2^-8,
# the unit roundoff of bf16, a row y_i of the oracle and the GPU's row x_i:
#   every row: the GPU rounds its fp32 result to bf16 once, |error| <= u|y_i|;
#   O, dV (prefill): each probability P_ij is rounded to bf16 before the PV or
#     P^T dO product, relative error <= u, independent across the terms; their
#     effect has RMS u/sqrt(3) * r_i with r_i = sqrt(sum_j (P_ij |v_j|)^2) (the
#     oracle's error scale of the row);
#   dQ, dK: P and then dS are rounded to bf16 (r_i as above over the terms
#     dS_ij |k_j|, resp. dS_ij |q_i|), and dS = P (dP - D) subtracts two fp32 dot
#     products of d terms, whose rounding (RMS about 2^-24 sqrt(d) times the sum
#     of the terms' magnitudes) is not small next to dP - D where a row's
#     probability sits on one key; c_i sums those magnitudes the same way;
#   decode O: the decode kernel keeps probabilities in fp32, so only the
#     output rounding and fp32 sums (well below 2^-12 relative) remain.
# The bound allows 4 times each RMS term (about 7 standard deviations), so a
# row within it is right to rounding; a row 10% wrong exceeds it unless the row
# itself is a near-total cancellation.  Each test prints the worst ratio of
# error to bound.
U_BF16 = 2.0 ** -8


def row_bounds(name, y, r=None, c=None):
    """Per-row bound (last axis = row elements) for tensor `name`."""
    y = np.asarray(y, dtype=np.float64)
    yn = np.linalg.norm(y, axis=-1)
    d = y.shape[-1]
    if name == "o_decode":
        return (U_BF16 + 2.0 ** -12) * yn + 1e-30
    b = U_BF16 * yn + 4 * U_BF16 * np.asarray(r, dtype=np.float64) + 1e-30
    if name in ("dq", "dk"):
        b = b + 4 * 2.0 ** -24 * math.sqrt(d) * np.asarray(c, dtype=np.float64)
    return b


def check_rows(name, x, y, what="", r=None, c=None):
    """Asserts every row of x within its bound against the oracle's y
    (name: "o", "dv", "dq", "dk" with the oracle's error scales r (and c), or
    "o_decode"); rows the oracle did not compute (NaN) are skipped.  Prints
    the worst ratio of error to bound and the worst plain relative error."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    dd = y.shape[-1]
    x2, y2 = x.reshape(-1, dd), y.reshape(-1, dd)
    ok = np.isfinite(y2).all(-1)
    bound = row_bounds(name, y2, None if r is None else np.asarray(r).reshape(-1),
                       None if c is None else np.asarray(c).reshape(-1))
    err = np.linalg.norm(x2 - y2, axis=-1)
    ratio = np.where(ok, err / bound, 0.0)
    rel = np.where(ok, err / np.maximum(np.linalg.norm(y2, axis=-1), 1e-300), 0.0)
    i = int(np.argmax(ratio))
    print(f"ROWS {what} {name}: worst error/bound {ratio[i]:.3f} (row {i}, error {err[i]:.3e}, "
          f"|y| {np.linalg.norm(y2[i]):.3e}); worst relative error {rel.max():.3e}")
    assert ratio[i] <= 1.0, f"{what} {name}: row {i} error {err[i]:.3e} exceeds its bound {bound[i]:.3e}"
    return float(ratio[i])


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


def _listing(mask, gpu_keep, ora_keep, ora_T, gpu_ts=None):
    out = []
    for idx in zip(*np.nonzero(mask)):
        e = tuple(int(x) for x in idx) + (float(ora_T[idx]), int(gpu_keep[idx]), int(ora_keep[idx]))
        if gpu_ts is not None:
            e += (float(np.exp2(gpu_ts[idx])),)
        out.append(e)
    return out


def decision_report(gpu_keep, ora_keep, ora_T, legal, band=BAND, what="", gpu_ts=None):
    """Forward / decode rule.  Returns (n_bad, n_near, near_list): mismatches
    outside the band, and the tiles in the band, each listed as
    (index..., T_oracle, gpu decision, oracle decision[, T_gpu]).  The band
    tiles are printed."""
    legal = np.broadcast_to(legal, gpu_keep.shape)
    near = legal & np.isfinite(ora_T) & (np.abs(ora_T - 1.0) <= band)
    bad = legal & (gpu_keep != ora_keep) & ~near
    near_list = _listing(near, gpu_keep, ora_keep, ora_T, gpu_ts)
    print(f"BAND {what}: {len(near_list)} tiles with |T-1| <= {band:g} "
          f"(index, T_oracle, gpu, oracle[, T_gpu]): {near_list}")
    if bad.any():
        print(f"MISMATCH {what}: {_listing(bad, gpu_keep, ora_keep, ora_T, gpu_ts)[:20]}")
    return int(bad.sum()), int(near.sum()), near_list


def bwd_decision_check(gpu_keep, ora_keep, ora_T, legal, what="", gpu_ts=None):
    """Backward rule: the GPU's decisions must equal the free-running
    oracle's on every legal tile (no band exclusion).  Band tiles are printed
    as a diagnostic.  Returns the number of band tiles."""
    legal = np.broadcast_to(legal, gpu_keep.shape)
    near = legal & np.isfinite(ora_T) & (np.abs(ora_T - 1.0) <= BAND)
    bad = legal & (gpu_keep != ora_keep)
    print(f"BAND {what} (diagnostic): {int(near.sum())} tiles with |T-1| <= {BAND:g}: "
          f"{_listing(near, gpu_keep, ora_keep, ora_T, gpu_ts)}")
    assert not bad.any(), (f"{what}: backward decisions differ on {int(bad.sum())} tiles "
                           f"(index, T_oracle, gpu, oracle[, T_gpu]): "
                           f"{_listing(bad, gpu_keep, ora_keep, ora_T, gpu_ts)[:20]}")
    return int(near.sum())


def nesting_check(fwd_keep, bwd_keep, legal, fwd_ts, bwd_ts, what=""):
    """Backward support nested in forward's (backward paragraph), on the GPU's
    own decisions over every legal tile.  A tile kept by backward and skipped
    by forward can only arise where both tests sit on the threshold (the
    backward normalizer is the forward's final one, never smaller than the
    running one), and there fp32 rounding of the two forms decides; such a
    tile must have both GPU statistics within the band, and is printed.
    Returns the list of violations."""
    legal = np.broadcast_to(legal, fwd_keep.shape)
    viol = legal & (bwd_keep == 1) & (fwd_keep == 0)
    lb = np.log2(1.0 + BAND)
    out = [tuple(int(x) for x in idx) + (float(np.exp2(fwd_ts[idx])), float(np.exp2(bwd_ts[idx])))
           for idx in zip(*np.nonzero(viol))]
    print(f"NESTING {what}: {len(out)} backward-kept tiles that forward skipped (index, T_fwd, T_bwd): {out}")
    for e in out:
        tf, tb = np.log2(e[-2]), np.log2(e[-1])
        assert abs(tf) <= lb and abs(tb) <= lb, f"{what}: nesting violated outside the band at {e}"
    return out


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
