"""GPU parity of attn_fwd_merge: results over disjoint key shards, combined.

Each head's keys and values are cut into G shards (ragged lengths); the
forward runs on each shard with attn_fwd_ex (N queries against the shard's
keys), and attn_fwd_merge combines the G (O_s, lse_s) into the result over
all keys, the exact merge of page 3 "OpenAI Triton from introduction to model
practice" section 1.1 (block maxima and sums) through the log-sum-exp that
section 5 stores.  That is the one-GPU half of splitting a long key/value
cache over GPUs.  The merged O and lse are compared element by element with
the fp64 oracle over the whole key set, at the forward's bars: the shard
outputs are rounded to the element type before the merge, which adds at most
one more rounding of that size.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from test_parity import check

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _attn():
    import attention_attn_fwd_07_amd as attn
    return attn


def _shards(Nk, G, seed):
    """G ragged, non-empty, contiguous key ranges covering 0 .. Nk - 1."""
    r = np.random.default_rng(seed)
    cuts = np.sort(r.choice(np.arange(1, Nk), size=G - 1, replace=False)) if G > 1 else []
    edges = [0, *[int(c) for c in cuts], Nk]
    return [(edges[i], edges[i + 1]) for i in range(G)]


def _merged(q, k, v, scale, shards, order=None):
    attn = _attn()
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    parts = [attn.fwd(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), scale)
             for a, b in shards]
    if order is not None:
        parts = [parts[i] for i in order]
    o, lse = attn.merge([p[0] for p in parts], [p[1] for p in parts])
    torch.cuda.synchronize()
    return o, lse, parts


CASES = [  # (dtype, d, N, Nk, G)
    ("bf16", 128, 1, 5000, 2), ("bf16", 64, 100, 3000, 3), ("f16", 128, 300, 1000, 7),
    ("f16", 64, 17, 64, 5), ("f32", 128, 40, 900, 4), ("f32", 64, 1, 3, 3),
    ("bf16", 128, 1000, 2048, 2), ("bf16", 64, 2, 65, 64)]


@pytest.mark.parametrize("dtype,d,N,Nk,G", CASES,
                         ids=[f"{a}-d{b}-N{c}-Nk{e}-G{f}" for a, b, c, e, f in CASES])
def test_merge_of_key_shards(dtype, d, N, Nk, G):
    q, k, v = datagen.make_qkv_kv(2, 2, N, Nk, d, dtype, 900 + N + G,
                                  hot_frac=0.02 if dtype != "f32" else 0.0, hot_mult=8.0)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse, _ = _merged(q, k, v, scale, _shards(Nk, G, 901 + G))
    o_ref, lse_ref = oracle.attention(q, k, v, scale)
    check(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, dtype,
          f"merge {dtype} d{d} N{N} Nk{Nk} G{G}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_of_one_part_is_that_part(dtype):
    """One part: weight 1 and sum 1, so O and lse come back bit for bit."""
    attn = _attn()
    q, k, v = (t.to(DEV) for t in datagen.make_qkv(1, 3, 200, 128, dtype, 910))
    o1, l1 = attn.fwd(q, k, v)
    o, lse = attn.merge([o1], [l1])
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, l1)


def test_merge_order_and_determinism():
    """The parts in another order give the same result up to fp32 rounding
    (both against the oracle), and repeated calls are bit-identical."""
    q, k, v = datagen.make_qkv_kv(1, 2, 64, 4000, 128, "bf16", 920)
    scale = 0.088
    shards = _shards(4000, 6, 921)
    o1, l1, _ = _merged(q, k, v, scale, shards)
    o2, l2, _ = _merged(q, k, v, scale, shards, order=[5, 3, 1, 0, 2, 4])
    o3, l3, _ = _merged(q, k, v, scale, shards)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    o_ref, lse_ref = oracle.attention(q, k, v, scale)
    for o, lse in ((o1, l1), (o2, l2)):
        check(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, "bf16",
              "merge order")
    assert float((l1 - l2).abs().max()) <= 1e-5


def test_merge_nan_part_poisons_its_rows_only():
    attn = _attn()
    q, k, v = (t.to(DEV) for t in datagen.make_qkv_kv(1, 2, 3, 300, 64, "bf16", 930))
    k[0, 0, 250, 5] = float("nan")
    parts = [attn.fwd(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous())
             for a, b in ((0, 200), (200, 300))]
    o, lse = attn.merge([p[0] for p in parts], [p[1] for p in parts])
    torch.cuda.synchronize()
    assert bool(torch.isnan(o[0, 0]).all()) and bool(torch.isnan(lse[0, 0]).all())
    assert bool(torch.isfinite(o[0, 1]).all()) and bool(torch.isfinite(lse[0, 1]).all())


def test_merge_binding_rejects_bad_parts():
    attn = _attn()
    o = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 1, 8, device=DEV)
    with pytest.raises(ValueError):
        attn.merge([o, o.float()], [lse, lse])            # mixed dtypes
    with pytest.raises(ValueError):
        attn.merge([o], [lse[:, :, :4]])                  # wrong lse shape
    with pytest.raises(ValueError):
        attn.merge([o] * 65, [lse] * 65)                  # more parts than ATTN_MAX_SPLITS
    with pytest.raises(ValueError):
        attn.merge([o], [lse], o=o)                       # output aliases a part
    with pytest.raises(ValueError):
        attn.merge([o.cpu()], [lse.cpu()])                # host tensors
    with pytest.raises(ValueError):
        attn.merge([o], [lse], o=torch.empty_like(o).cpu())  # output on the host
    with pytest.raises(ValueError):
        attn.merge([o], [lse], lse=torch.empty(1, 1, 8, device=DEV, dtype=torch.float16))
