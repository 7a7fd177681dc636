"""Plain float64 gradients of attention (test infrastructure only).

What the backward pass computes. [FA-Fill Exercise 5]: the forward pass keeps only O and
the row statistics m (row maximum) and l (row sum of exp(s - m)); the backward pass
recomputes P_ij = exp(S_ij - m_i) / l_i block by block from them and accumulates
dV_j = sum_i P_ij^T dO_i. [CS349E-L11] (its note on FlashAttention-2's non-matmul work):
only one number per row is kept, the log-sum-exp L = m + ln(l), so P_ij = exp(S_ij - L_i).
[FA-Simplified §7] lists the backward pass (recomputation plus blockwise gradients) as the
first extension without giving dQ and dK. They follow from the definition
O = softmax(S) V, S = scale Q K^T by the chain rule, and that is what is written here:

    dP = dO V^T
    dS_ij = P_ij (dP_ij - D_i),    D_i = sum_j P_ij dP_ij
    dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO

With grouped K/V heads, dK and dV of a K/V head sum over the query heads that read it;
under the causal mask the masked P_ij are 0 and contribute nothing.
"""
from __future__ import annotations

import numpy as np

from .attention import causal_last_key, kv_head_of, scores_fp64, NEG_INF


def _probabilities(q, k, scale, rows, Nq, causal):
    """P rows of one head: the definition's softmax of the (masked) scaled scores, float64."""
    s = scores_fp64(q[rows], k, scale)
    if causal:
        last = causal_last_key(rows, Nq, k.shape[0])
        s = np.where(np.arange(k.shape[0])[None, :] <= last[:, None], s, NEG_INF)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def attention_backward_fp64(q, k, v, do, scale, causal: bool = False, row_block: int = 512):
    """Gradients of O = softmax(scale Q K^T) V: returns (dq, dk, dv, lse, delta).

    q, do [B, H, Nq, d]; k, v [B, H_kv, Nk, d] (query head h reads K/V head
    ``kv_head_of(h, H, H_kv)``). dq has q's shape, dk and dv k's. ``lse`` [B, H, Nq] is
    m + ln(l) of each row and ``delta`` [B, H, Nq] is D_i = sum_j P_ij dP_ij. Rows are
    taken ``row_block`` at a time (every block sees all keys, so each P row is complete);
    that bounds this reference's memory and changes no arithmetic.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    assert v.shape == k.shape and do.shape[:3] == q.shape[:3]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros((B, H_kv, Nk, v.shape[-1]))
    lse = np.empty((B, H, Nq))
    delta = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            hk = kv_head_of(h, H, H_kv)
            K, V = k[b, hk], v[b, hk]
            for r0 in range(0, Nq, row_block):
                rows = np.arange(r0, min(Nq, r0 + row_block))
                P, m, l = _probabilities(q[b, h], K, scale, rows, Nq, causal)
                dO = do[b, h, rows]
                dP = dO @ V.T
                D = (P * dP).sum(axis=1)
                dS = P * (dP - D[:, None])
                dq[b, h, rows] = float(scale) * (dS @ K)
                dk[b, hk] += float(scale) * (dS.T @ q[b, h, rows])
                dv[b, hk] += P.T @ dO
                lse[b, h, rows] = m + np.log(l)
                delta[b, h, rows] = D
    return dq, dk, dv, lse, delta


def dv_from_statistics_blocked(q, k, do, m, l, scale, block: int):
    """[FA-Fill Exercise 5]: dV of one head rebuilt block by block from the stored m and l.

    For every key block j and query block i: S_ij = scale Q_i K_j^T,
    P_ij = exp(S_ij - m_i) / l_i with the forward pass's global statistics (not the
    block's), and dV_j += P_ij^T dO_i. q, do [Nq, d]; k [Nk, d]; m, l [Nq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    dv = np.zeros((k.shape[0], do.shape[1]))
    for j0 in range(0, k.shape[0], block):
        for i0 in range(0, q.shape[0], block):
            s = float(scale) * (q[i0:i0 + block] @ k[j0:j0 + block].T)
            p = np.exp(s - m[i0:i0 + block, None]) / l[i0:i0 + block, None]
            dv[j0:j0 + block] += p.T @ do[i0:i0 + block]
    return dv


def attention_loss_fp64(q, k, v, do, scale, causal: bool = False) -> float:
    """sum(O * dO): the scalar whose gradients are dq, dk, dv (used by the finite-difference pin)."""
    from .attention import attention_fp64
    o = attention_fp64(q, k, v, scale, causal=causal)
    return float(np.sum(o * np.asarray(do, dtype=np.float64)))
