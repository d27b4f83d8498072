"""Gradients of the attention forward, in float64 (test infrastructure).

Page 3 section 6 wraps the fused forward in an autograd function whose
forward saves (q, k, v, o, lse) for a backward pass (the backward kernel
itself is not shown).  The gradients it must produce are those of the plain
definition, O = softmax(scale * Q K^T) V per (b, h), by the chain rule.  With
P the softmax weights and dO the gradient of the loss with respect to O:

1. dV = P^T dO                      (O = P V is linear in V)
2. dP = dO V^T                      (and linear in P)
3. D_i = sum_c dO_ic O_ic           (= sum_j P_ij dP_ij, since O_i = sum_j P_ij V_j)
4. dS = P * (dP - D)                (the softmax Jacobian: dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik))
5. dQ = scale * dS K,  dK = scale * dS^T Q   (S = scale * Q K^T)

Causal: masked scores have P_ij = 0 exactly, so they receive no gradient and
pass none on; the same formulas hold with the masked P.

Query rows are processed in chunks (dQ rows are independent; dK and dV sum
the chunks' contributions), with numpy matrix products as the only library
primitive.  Inputs are used as given, upcast to float64.
"""
from __future__ import annotations

import numpy as np

from .definition import ROW_CHUNK, _as64, _default_workers, _run_tasks

__all__ = ["attention_backward"]


def _head_backward(q, k, v, do, scale, causal, row_chunk):
    """dq, dk, dv for one head: q, k, v, do are [N, d] float64."""
    N = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    cols = np.arange(N)[None, :]
    for i0 in range(0, N, row_chunk):
        i1 = min(N, i0 + row_chunk)
        s = float(scale) * (q[i0:i1] @ k.T)                  # scores of the chunk's rows
        if causal:
            s[cols > np.arange(i0, i1)[:, None]] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)                     # P, the softmax weights
        o = p @ v                                             # O of these rows
        dv += p.T @ do[i0:i1]                                 # 1. dV = P^T dO
        dp = do[i0:i1] @ v.T                                  # 2. dP = dO V^T
        dd = (do[i0:i1] * o).sum(axis=1, keepdims=True)       # 3. D = rowsum(dO * O)
        ds = p * (dp - dd)                                    # 4. dS = P * (dP - D)
        dq[i0:i1] = float(scale) * (ds @ k)                   # 5. dQ = scale dS K
        dk += float(scale) * (ds.T @ q[i0:i1])                #    dK = scale dS^T Q
    return dq, dk, dv


def attention_backward(q, k, v, do, scale: float, *, causal: bool = False,
                       workers: int | None = None, row_chunk: int = ROW_CHUNK):
    """dq, dk, dv (float64, shape [B, H, N, d]) of O = softmax(scale Q K^T) V
    for the upstream gradient ``do`` of O.  ``causal``: query i sees keys 0..i."""
    q, k, v, do = (_as64(x) for x in (q, k, v, do))
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape or do.shape != q.shape:
        raise ValueError(f"shape mismatch: q{q.shape} k{k.shape} v{v.shape} do{do.shape}")
    B, H = q.shape[:2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)

    def run(task):
        b, h = task
        dq[b, h], dk[b, h], dv[b, h] = _head_backward(q[b, h], k[b, h], v[b, h], do[b, h],
                                                      scale, causal, row_chunk)

    _run_tasks(run, [(b, h) for b in range(B) for h in range(H)], workers)
    return dq, dk, dv
