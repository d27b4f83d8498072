"""The plain definition of attention forward, in float64 (test infrastructure).

What it computes, per batch b, head h and query row i < N, for keys j < Nk
(Nk = N for self-attention; a few queries against a long key/value history,
Nk > N, is how generation scores each new position against all cached keys,
the bandwidth-bound inference case of page 3 section 4):

1. s_ij  = scale * sum_c Q[b,h,i,c] * K[b,h,j,c]
   (page 3, section 3, the decoder layer's scores: Q times K transposed divided
   by sqrt(head_dim); page 3 section 1.2 figure 1-A step 5.  The scale is the
   caller's argument; the workloads pass 1/sqrt(d)).
2. m_i   = max_j s_ij
3. p_ij  = exp(s_ij - m_i)
   (the max-subtracted softmax of page 4's softmax kernel: subtract the row
   max, exponentiate, sum, divide.)
4. l_i   = sum_j p_ij
5. O[b,h,i,:] = (sum_j p_ij * V[b,h,j,:]) / l_i
   (page 3 section 3: softmax of the scores times V.)
6. lse[b,h,i] = m_i + ln l_i
   (page 3 section 5: the kernel also stores the log-sum-exp of the scaled
   scores, max plus log of the exp-sum.)

Causal variant (``causal=True``): query row i sees only keys j <= i.  Page 1
section 4 notes that real kernels add a causal mask; page 3 section 3's
decoder layer fills masked scores with -1e9 before the softmax, and page 3
section 5's autograd wrapper passes a ``causal`` flag to the forward.  Here the
masked scores are excluded outright (set to -inf, so their exponentials are
exactly zero); with -1e9 they would underflow to zero in float64 anyway for
any finite scores of moderate size.  Every row keeps at least key 0, so m_i is
finite.

The full N x N score matrix is materialised, one chunk of query rows at a time
so that memory stays bounded (a 256 x 65536 fp64 chunk is 128 MiB).  The matrix
products and the elementwise exp/log are numpy library primitives; there is no
blocking, fusion or reordering of the definition beyond that row chunking.
Query rows are independent, so chunking changes nothing mathematically; only
the BLAS library's own summation order may differ between chunk shapes (a few
float64 ulps).

Inputs are used exactly as given, upcast to float64: callers pass the
dtype-rounded tensors, so input rounding is shared with the GPU path.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # keep one BLAS thread per task when a thread pool drives the work
    from threadpoolctl import threadpool_limits
except ImportError:  # pragma: no cover - threadpoolctl is installed here
    threadpool_limits = None

ROW_CHUNK = 256


def _as64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: go through float64 on the CPU
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def scores(q, k, scale: float) -> np.ndarray:
    """Step 1 for one head: s = scale * q k^T, q [M, d], k [N, d] -> [M, N]."""
    q = _as64(q)
    k = _as64(k)
    return float(scale) * (q @ k.T)


def _rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, rows=None):
    """Steps 1-6 for a block of query rows of one head.

    q [M, d], k [N, d], v [N, dv] (float64).  Returns (o [M, dv], lse [M]).
    ``rows`` (causal only): the absolute query index of each of the M rows;
    row r then sees keys j <= rows[r] only.
    """
    s = float(scale) * (q @ k.T)            # 1. scaled scores, [M, N]
    if rows is not None:                    #    causal: drop keys after the query
        s[np.arange(k.shape[0])[None, :] > np.asarray(rows)[:, None]] = -np.inf
    m = s.max(axis=1, keepdims=True)        # 2. row max
    p = np.exp(s - m)                       # 3. max-subtracted exponentials
    l = p.sum(axis=1, keepdims=True)        # 4. row sums
    o = (p @ v) / l                         # 5. normalised weighted sum of V
    lse = m[:, 0] + np.log(l[:, 0])         # 6. log-sum-exp of the scores
    return o, lse


def softmax_probs(q, k, scale: float, causal: bool = False) -> np.ndarray:
    """The attention weights p_ij / l_i for one head (small shapes only)."""
    s = scores(q, k, scale)
    if causal:
        s[np.triu(np.ones(s.shape, dtype=bool), 1)] = -np.inf
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=1, keepdims=True)


def _default_workers() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _check_shapes(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool) -> None:
    """q [B, H, N, d], k [B, H, Nk, d], v [B, H, Nk, dv]; Nk >= 1 when N > 0
    (a softmax over no keys is undefined); causal needs Nk = N."""
    if (q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or k.shape[:2] != q.shape[:2]
            or k.shape[3] != q.shape[3] or v.shape[:3] != k.shape[:3]):
        raise ValueError(f"shape mismatch: q{q.shape} k{k.shape} v{v.shape}")
    if k.shape[2] == 0 and q.shape[2] > 0 and q.shape[0] * q.shape[1] > 0:
        raise ValueError("no keys: the softmax over an empty row is undefined")
    if causal and k.shape[2] != q.shape[2]:
        raise ValueError("the causal mask is defined for equal query and key lengths")


def attention(q, k, v, scale: float, *, causal: bool = False, workers: int | None = None,
              row_chunk: int = ROW_CHUNK):
    """O and lse for q [B, H, N, d], k [B, H, Nk, d], v [B, H, Nk, dv] (any
    float input dtype; Nk = N for self-attention).

    ``causal``: query row i attends keys 0..i only (needs Nk = N).

    Returns (o, lse): float64 arrays of shape [B, H, N, dv] and [B, H, N].
    Work is split into (b, h, row-chunk) tasks on a thread pool with BLAS held
    to one thread per task; every task evaluates the same plain definition.
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    _check_shapes(q, k, v, causal)
    B, H, N, _ = q.shape
    o = np.empty((B, H, N, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    if N == 0:
        return o, lse
    tasks = [(b, h, i0) for b in range(B) for h in range(H)
             for i0 in range(0, N, row_chunk)]

    def run(task):
        b, h, i0 = task
        i1 = min(N, i0 + row_chunk)
        if causal:
            o[b, h, i0:i1], lse[b, h, i0:i1] = _rows(q[b, h, i0:i1], k[b, h], v[b, h], scale,
                                                     np.arange(i0, i1))
        else:
            o[b, h, i0:i1], lse[b, h, i0:i1] = _rows(q[b, h, i0:i1], k[b, h], v[b, h], scale)

    _run_tasks(run, tasks, workers)
    return o, lse


def attention_rows(q, k, v, scale: float, index, *, causal: bool = False,
                   workers: int | None = None):
    """O and lse for selected query rows only.

    ``index`` is an integer array of shape [R, 3] holding (b, h, i) triples.
    Returns (o [R, d], lse [R]) in float64.  Each row needs its head's full K
    and V, and rows are independent, so these values are exactly those of
    ``attention`` at the same positions.
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    _check_shapes(q, k, v, causal)
    index = np.asarray(index, dtype=np.int64).reshape(-1, 3)
    R = index.shape[0]
    o = np.empty((R, v.shape[-1]), dtype=np.float64)
    lse = np.empty(R, dtype=np.float64)
    groups: dict[tuple[int, int], list[int]] = {}
    for r, (b, h, _) in enumerate(index):
        groups.setdefault((int(b), int(h)), []).append(r)
    tasks = []
    for (b, h), rs in groups.items():
        for c0 in range(0, len(rs), ROW_CHUNK):
            tasks.append((b, h, rs[c0:c0 + ROW_CHUNK]))

    def run(task):
        b, h, rs = task
        rows = index[rs, 2]
        if causal:
            o[rs], lse[rs] = _rows(q[b, h, rows], k[b, h], v[b, h], scale, rows)
        else:
            o[rs], lse[rs] = _rows(q[b, h, rows], k[b, h], v[b, h], scale)

    _run_tasks(run, tasks, workers)
    return o, lse


def _run_tasks(run, tasks, workers):
    workers = _default_workers() if workers is None else max(1, int(workers))
    if workers == 1 or len(tasks) <= 1:
        for t in tasks:
            run(t)
        return
    ctx = threadpool_limits(limits=1) if threadpool_limits is not None else None
    try:
        if ctx is not None:
            ctx.__enter__()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(run, t) for t in tasks]:
                f.result()
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
