"""GPU parity of the split-KV path (attn_fwd_splitkv).

Each split of a head's keys produces a normalised partial output and its
log-sum-exp; a merge kernel combines them as page 3 section 1.1 combines the
per-block maxima and sums of a long softmax row.  The merged result is held to
the same bars as the single-pass path against the fp64 oracle, and to the
single-pass result itself (the two differ only by fp32 summation order and
the output rounding).
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from test_parity import TOL, check

pytestmark = pytest.mark.gpu


def _attn():
    import attention_attn_fwd_07_amd as attn
    return attn


def splitkv_parity(q, k, v, scale, dtype, splits, what, kernel=None, monkeypatch=None):
    attn = _attn()
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = attn.fwd_splitkv(qd, kd, vd, scale, splits=splits)
    o1, l1 = attn.fwd(qd, kd, vd, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, scale)
    o64, l64 = o.cpu().double().numpy(), lse.cpu().double().numpy()
    check(o64, l64, o_ref, lse_ref, dtype, what)
    # against the single pass: the same bar, and lse within fp32 rounding
    assert np.abs(o64 - o1.cpu().double().numpy()).max() <= TOL[dtype]["maxabs"]
    assert np.abs(l64 - l1.cpu().double().numpy()).max() <= 1e-5
    return o, lse


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 64), ("f32", 128),
                                     ("bf16", 64), ("f16", 128)])
@pytest.mark.parametrize("N,splits", [(1, 3), (63, 2), (64, 4), (65, 2), (1000, 3), (1000, 64),
                                      (2049, 7), (1000, 1), (200, 1)])
def test_splitkv_shapes(dtype, d, N, splits):
    """Shapes and split counts, among them a single split on grids where the
    plain path would split keys inside each block (the split-KV path must
    still write the partial results its merge reads)."""
    q, k, v = datagen.make_qkv(1, 2, N, d, dtype, seed=600 + N + splits)
    splitkv_parity(q, k, v, 1.0 / math.sqrt(d), dtype, splits,
                   f"splitkv {dtype} d={d} N={N} splits={splits}")


@pytest.mark.parametrize("kernel", ["pingpong", "pipelined", "pipelined2"])
def test_splitkv_both_kernels_hot_keys(kernel, monkeypatch):
    monkeypatch.setenv("ATTN_FWD_KERNEL", kernel)
    q, k, v = datagen.make_qkv(1, 2, 3000, 128, "bf16", seed=61, hot_frac=0.01, hot_mult=8.0)
    splitkv_parity(q, k, v, 1.0 / math.sqrt(128), "bf16", 5, f"splitkv hot keys {kernel}")


def test_splitkv_long_single_head():
    """B=1 H=2 N=16384 d=128 fp16 (the long-sequence shape with few heads that
    leaves most compute units idle in one pass), 8 splits, sampled rows."""
    attn = _attn()
    q, k, v = datagen.make_qkv(1, 2, 16384, 128, "f16", seed=62, mult=0.5)
    dev = torch.device("cuda:0")
    o, lse = attn.fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), 1 / math.sqrt(128), splits=8)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = [(0, h, int(i)) for h in range(2) for i in rng.choice(16384, 48, replace=False)]
    rows += [(0, h, i) for h in range(2) for i in (0, 1, 8191, 16383)]
    idx = np.array(rows)
    o_ref, lse_ref = oracle.attention_rows(q, k, v, 1 / math.sqrt(128), idx)
    o64, l64 = o.cpu().double().numpy(), lse.cpu().double().numpy()
    check(o64[idx[:, 0], idx[:, 1], idx[:, 2]], l64[idx[:, 0], idx[:, 1], idx[:, 2]], o_ref,
          lse_ref, "f16", "splitkv B1 H2 N16384 d128")


def test_splitkv_strided_and_plan():
    """Strided inputs and a reused plan with a caller-owned workspace."""
    attn = _attn()
    q, k, v = datagen.make_qkv(2, 3, 777, 64, "bf16", seed=63)
    dev = torch.device("cuda:0")
    qd = q.to(dev).transpose(1, 2).contiguous().transpose(1, 2)
    kd, vd = k.to(dev), v.to(dev)
    o = torch.empty(q.shape, dtype=q.dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    nbytes = attn.splitkv_workspace_size(2, 3, 777, 64, 6)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    p = attn.plan(qd, kd, vd, o, lse, 0.125, splits=6, workspace=ws)
    p()
    p()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, 0.125)
    check(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, "bf16",
          "splitkv strided plan")


def test_splitkv_rejects_causal_and_small_workspace():
    attn = _attn()
    q = torch.zeros(1, 1, 256, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    ws = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        attn.plan(q, q, q, o, None, 0.125, splits=2, workspace=ws)()
    ws = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        attn.plan(q, q, q, o, None, 0.125, causal=True, splits=2, workspace=ws)()
