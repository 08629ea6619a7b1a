"""Brute-force dense causal softmax attention in fp64 (numpy).

TEST INFRASTRUCTURE ONLY (a second, independent reference used to pin the
oracle).  This is the full-attention operator that MALA reduces to as tau
goes to 0 (MALA digest, savings paragraph): every causal interaction is
scored, normalized and used; no tiles, no online rescaling.
"""
import numpy as np


def scores(q, k, scale):
    """s[i, j] = scale * <q_i, k_j>, with -inf above the diagonal (j > i)."""
    L = q.shape[0]
    s = scale * (q @ k.T)
    s[np.triu_indices(L, 1)] = -np.inf
    return s


def fwd_head(q, k, v, scale, key_mask=None):
    """O and lse (natural log) of dense causal attention for one head.
    key_mask [L, L] bool, optional: restrict each row to the keys marked True."""
    s = scores(q, k, scale)
    if key_mask is not None:
        s = np.where(key_mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=1, keepdims=True)
    return (p @ v) / z, (m + np.log(z))[:, 0]


def probs_head(q, k, scale):
    s = scores(q, k, scale)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=1, keepdims=True)


def bwd_head(q, k, v, do, scale):
    """Exact gradients of sum(dO * O) for dense causal attention (one head).

    With P = softmax(S), S = scale * Q K^T (causal):
      dV = P^T dO;  dP = dO V^T;  dS = P * (dP - rowsum(dO * O));
      dQ = scale * dS K;  dK = scale * dS^T Q.
    """
    p = probs_head(q, k, scale)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    D = (do * o).sum(axis=1, keepdims=True)
    ds = p * (dp - D)
    return scale * ds @ k, scale * ds.T @ q, dv


def fwd(q, k, v, scale):
    B, H, L, d = q.shape
    o = np.zeros((B, H, L, d))
    lse = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = fwd_head(q[b, h], k[b, h], v[b, h], scale)
    return o, lse


def bwd(q, k, v, do, scale):
    B, H, L, d = q.shape
    out = [np.zeros((B, H, L, d)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            g = bwd_head(q[b, h], k[b, h], v[b, h], do[b, h], scale)
            for a, x in zip(out, g):
                a[b, h] = x
    return tuple(out)
