"""The online-softmax recurrence, in float64 (test infrastructure).

This is the one-pass method the pages build (page 1 section 4, "online softmax
three-piece set"; page 3 section 1.2 figure 1-A steps 3-7 and section 5
figure 5): K/V are visited in blocks of ``block_n`` keys while each query row
keeps a running max m, a running exp-sum l and an accumulator acc.  For each
key block:

    m_new = max(m, rowmax(S_block))
    p     = exp(S_block - m_new)
    alpha = exp(m - m_new)
    l     = alpha * l + rowsum(p)
    acc   = alpha * acc + p @ V_block
    m     = m_new

and at the end O = acc / l and lse = m + ln l.  m starts at -inf, l and acc at
zero (page 1's initial values).  A final partial block simply holds fewer keys,
which is what masking padded keys to -inf achieves (page 4's softmax kernel
pads with -inf so that exp of a pad is zero).

With ``causal=True`` the scores of keys after the query are -inf inside each
block (page 1 section 4's causal mask), so a block wholly after a query row
adds nothing to it: p = 0 and, with m already finite from key 0, alpha = 1.

In exact arithmetic this equals the two-pass definition in ``definition``; the
oracle tests use it only to pin that invariant, for several block sizes,
including sizes that do not divide N.
"""
from __future__ import annotations

import numpy as np


def attention_online(q, k, v, scale: float, block_n: int, causal: bool = False):
    """O, lse for q [B, H, N, d], k [B, H, Nk, d], v [B, H, Nk, dv] via the
    blockwise online recurrence over the Nk keys (causal needs Nk = N)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if block_n < 1:
        raise ValueError("block_n must be >= 1")
    B, H, N, _ = q.shape
    Nk = k.shape[2]
    if causal and Nk != N:
        raise ValueError("the causal mask is defined for equal query and key lengths")
    o = np.empty((B, H, N, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            qh, kh, vh = q[b, h], k[b, h], v[b, h]
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, vh.shape[1]))
            for j0 in range(0, Nk, block_n):
                j1 = min(Nk, j0 + block_n)
                s = float(scale) * (qh @ kh[j0:j1].T)
                if causal:
                    s[np.arange(j0, j1)[None, :] > np.arange(N)[:, None]] = -np.inf
                m_new = np.maximum(m, s.max(axis=1))
                p = np.exp(s - m_new[:, None])
                alpha = np.exp(m - m_new)
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ vh[j0:j1]
                m = m_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = m + np.log(l)
    return o, lse
