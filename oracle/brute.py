"""Brute-force NumPy form of the Orthros attention step, for tiny sizes.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

It writes the two attention domains of "Orthros:阶段感知异构注意力精读笔记"
§2.3 (Eqs. (4)-(5)) as explicit T x T mask matrices and a dense softmax,
the matrix form of the definition, independent of the loop form in
oracle.c:

    M_swa[t, j]  = (j <= t) and (j >= t - w + 1)       window W_t, 0-based
    M_glob[P, j] = (j <= P)                            copy at original position P

Queries get the per-stream scale-offset of §2.2 (q * alpha + beta).  All
arithmetic in float64.
"""
import numpy as np


def _softmax_rows(s):
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def swa_mask(T, w):
    t = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (j <= t) & (j >= t - w + 1)


def prefill(q, q_out, out_pos, k, v, alpha, beta, alpha_out, beta_out, window, scale):
    """q [B,T,Hq,d], q_out [B,Hq,d], k/v [B,T,Hkv,d], alpha.. [Hq,d] (float64 arrays).

    Returns (o [B,T,Hq,d], o_out [B,Hq,d]).
    """
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    M = swa_mask(T, window)
    o = np.zeros_like(q)
    o_out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            K = k[b, :, g, :]
            V = v[b, :, g, :]
            Qh = q[b, :, h, :] * alpha[h] + beta[h]
            S = scale * (Qh @ K.T)
            S = np.where(M, S, -np.inf)
            o[b, :, h, :] = _softmax_rows(S) @ V
            qh = q_out[b, h] * alpha_out[h] + beta_out[h]
            s = scale * (K @ qh)
            keep = np.arange(T) <= out_pos[b]
            s = np.where(keep, s, -np.inf)
            o_out[b, h] = _softmax_rows(s[None, :])[0] @ V
    return o, o_out
