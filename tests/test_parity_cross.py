"""GPU parity with a key length of its own: N query rows against Nk key and
value rows (k and v of shape [B, H, Nk, d]).

The case that motivates it is generation: each new position is scored against
the whole cached history of keys and values, a 1 x Nk row of scores per head
(page 3 "OpenAI Triton from introduction to model practice", section 4, which
names it the bandwidth-bound case of inference).  The cases cover one query
against short, ragged and long key sets, a few queries against many keys, many
queries against few keys, every kernel the library can pick for the 16-bit
types (up to four query rows go to the decode kernel, which streams K and V
with plain loads and computes on the VALU; up to 128 rows to the pipelined
kernel), the split-KV path (with a workspace and with the library's static
one), the [B, N, H, d] layout, hot keys, and the decode workload whole
(B=1, H=32, one query against 65536 keys, d=128, bf16, in the launch
configuration bench.py times).  Every element of O and lse is compared with
the fp64 oracle at the bars of test_parity.
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


def _run(q, k, v, scale, splits=0, static=False, bshd=False):
    attn = _attn()
    if bshd:
        qd, kd, vd = (t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, k, v))
    else:
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    if splits and static:
        o = torch.empty(q.shape, dtype=q.dtype, device=DEV)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
        attn.attn_fwd_splitkv_static(qd, kd, vd, o, lse, scale, splits)
    elif splits:
        o, lse = attn.fwd_splitkv(qd, kd, vd, scale, splits=splits)
    else:
        o, lse = attn.fwd(qd, kd, vd, scale)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def _compare(dtype, d, B, H, N, Nk, seed, scale=None, splits=0, static=False, bshd=False,
             hot=False, what=""):
    kw = dict(hot_frac=0.01, hot_mult=8.0) if hot else {}
    q, k, v = datagen.make_qkv_kv(B, H, N, Nk, d, dtype, seed, **kw)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _run(q, k, v, scale, splits, static, bshd)
    assert o.shape == (B, H, N, d) and lse.shape == (B, H, N)
    o_ref, lse_ref = oracle.attention(q, k, v, scale)
    check(o, lse, o_ref, lse_ref, dtype, what)


SHAPES = [  # (N, Nk): one query, few queries, more queries than keys
    (1, 1), (1, 63), (1, 64), (1, 65), (1, 1000), (1, 4096),
    (3, 17), (4, 1999), (5, 3000), (17, 2049), (64, 333),
    (300, 77), (1000, 64), (129, 1), (2, 5)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,Nk", SHAPES, ids=[f"N{a}-Nk{b}" for a, b in SHAPES])
def test_cross_lengths(dtype, d, N, Nk):
    _compare(dtype, d, 1, 2, N, Nk, seed=100 + N + Nk + d, what=f"{dtype} d{d} N{N} Nk{Nk}")


KERNELS = ["pingpong", "pipelined", "pipelined2"]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,Nk", [(1, 777), (7, 2500), (260, 100), (513, 1030)])
def test_cross_lengths_every_kernel(kernel, d, N, Nk, monkeypatch):
    monkeypatch.setenv("ATTN_FWD_KERNEL", kernel)
    _compare("bf16", d, 2, 1, N, Nk, seed=200 + N + Nk, hot=True,
             what=f"{kernel} d{d} N{N} Nk{Nk}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("splits", [1, 3, 16, 64])
@pytest.mark.parametrize("N,Nk", [(1, 4096), (4, 1500), (200, 130), (1, 65)])
def test_cross_lengths_splitkv(dtype, splits, N, Nk):
    _compare(dtype, 128 if dtype == "f16" else 64, 2, 2, N, Nk, seed=300 + N + Nk + splits,
             splits=splits, what=f"{dtype} splits{splits} N{N} Nk{Nk}")


@pytest.mark.parametrize("N,Nk,splits", [(1, 8192, 8), (3, 1000, 5)])
def test_cross_lengths_splitkv_static(N, Nk, splits):
    _compare("bf16", 128, 1, 4, N, Nk, seed=400 + Nk, splits=splits, static=True,
             what=f"static N{N} Nk{Nk}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,Nk,splits", [(1, 3000, 0), (5, 2000, 4), (700, 90, 0)])
def test_cross_lengths_bshd(dtype, N, Nk, splits):
    _compare(dtype, 128, 2, 3, N, Nk, seed=500 + N, splits=splits, bshd=True,
             what=f"bshd {dtype} N{N} Nk{Nk}")


def test_cross_lengths_scale_of_either_sign():
    _compare("bf16", 64, 1, 2, 9, 1111, seed=601, scale=-0.3, what="negative scale")
    _compare("f32", 128, 1, 2, 9, 1111, seed=602, scale=0.4, what="scale 0.4")


SMALL_N = [(5, 1), (5, 63), (16, 64), (31, 65), (32, 257), (33, 4000), (64, 1111), (40, 200)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [0, 5])
@pytest.mark.parametrize("N,Nk", SMALL_N, ids=[f"N{a}-Nk{b}" for a, b in SMALL_N])
def test_few_query_rows(dtype, d, splits, N, Nk):
    """5 to 64 query rows (the pipelined kernel's 128-row blocks, whatever
    the grid), with and without key splits, hot keys."""
    _compare(dtype, d, 2, 2, N, Nk, seed=1000 + N + Nk + d, splits=splits, hot=True,
             what=f"few rows {dtype} d{d} N{N} Nk{Nk} S{splits}")


@pytest.mark.parametrize("key", [10, 70, 130, 200])
def test_few_rows_nan_key_poisons_its_head_only(key):
    """A NaN key anywhere in a head's keys (four different 64-key tiles)
    reaches every output row of that head and no other."""
    q, k, v = datagen.make_qkv_kv(1, 2, 20, 256, 128, "bf16", 1100 + key)
    k[0, 1, key, 3] = float("nan")
    o, lse = _run(q, k, v, 0.088)
    assert np.all(np.isnan(o[0, 1])) and np.all(np.isnan(lse[0, 1]))
    assert np.all(np.isfinite(o[0, 0])) and np.all(np.isfinite(lse[0, 0]))


@pytest.mark.parametrize("N", [1, 2, 3, 4, 20])
def test_decode_kernel_is_deterministic(N):
    """The same inputs give the same bits, with and without key splits."""
    attn = _attn()
    q, k, v = (t.to(DEV) for t in datagen.make_qkv_kv(2, 3, N, 2500, 128, "bf16", 700 + N))
    o1, l1 = attn.fwd(q, k, v)
    o2, l2 = attn.fwd(q, k, v)
    s1, m1 = attn.fwd_splitkv(q, k, v, splits=7)
    s2, m2 = attn.fwd_splitkv(q, k, v, splits=7)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(s1, s2) and torch.equal(m1, m2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("splits", [0, 5])
def test_decode_nan_key_poisons_its_head_only(dtype, splits):
    """A NaN in one key row of head 0 makes that head's outputs NaN (whole-row
    IEEE propagation, on both sides) and leaves head 1 finite, with and
    without key splits: the NaN key sits in one group of one wave of one
    split, and the block and split merges must carry it."""
    q, k, v = datagen.make_qkv_kv(1, 2, 2, 3000, 128, dtype, 801)
    k[0, 0, 1234, 7] = float("nan")
    o, lse = _run(q, k, v, 0.088, splits=splits)
    assert np.all(np.isnan(o[0, 0])) and np.all(np.isnan(lse[0, 0]))
    assert np.all(np.isfinite(o[0, 1])) and np.all(np.isfinite(lse[0, 1]))


@pytest.mark.parametrize("dtype,d", [("bf16", 128)])
def test_decode_longest_key_length(dtype, d):
    """One query per head against ATTN_MAX_N = 2^22 keys (the largest key
    length; row offsets up to 2^31 - 256 bytes at d = 128 bf16), plain and
    with 64 splits, every output against the oracle."""
    N, Nk = 1, 1 << 22
    q, k, v = datagen.make_qkv_kv(1, 1, N, Nk, d, dtype, 802)
    o_ref, lse_ref = oracle.attention(q, k, v, 0.1)
    for splits in (0, 64):
        o, lse = _run(q, k, v, 0.1, splits=splits)
        check(o, lse, o_ref, lse_ref, dtype, f"{dtype} d{d} Nk=2^22 splits={splits}")


def test_causal_needs_equal_lengths():
    attn = _attn()
    q, k, v = (torch.zeros(1, 1, n, 64, dtype=torch.bfloat16, device=DEV) for n in (4, 8, 8))
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, causal=True)
    with pytest.raises(ValueError):
        attn.fwd(q, k[:, :, :0], v[:, :, :0])
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, torch.zeros_like(q), torch.zeros(1, 1, 4, device=DEV), q)


def test_decode_workload_whole():
    """One query per head against 65536 cached keys (B=1, H=32, d=128, bf16),
    through the split-KV path with the split count bench.py uses, every
    output element against the oracle."""
    import bench
    w = datagen.DECODE
    q, k, v = datagen.make_qkv_kv(w["B"], w["H"], w["N"], w["Nk"], w["d"], w["dtype"], w["seed"])
    scale = float(np.float32(1.0 / np.sqrt(w["d"])))
    o, lse = _run(q, k, v, scale, splits=bench.decode_splits(w))
    o_ref, lse_ref = oracle.attention(q, k, v, scale)
    check(o, lse, o_ref, lse_ref, w["dtype"], w["name"])
    # the outputs lie in the convex hull of V's rows
    v64 = v.double().numpy()
    assert np.all(o >= v64.min(axis=2, keepdims=True) - 2e-2)
    assert np.all(o <= v64.max(axis=2, keepdims=True) + 2e-2)


NRANDOM = 60


def _random_case(i):
    rng = np.random.default_rng(9500 + i)
    dtype = ["bf16", "f16", "f32"][int(rng.integers(3))]
    d = [64, 128][int(rng.integers(2))]
    N = int(np.exp(rng.uniform(0.0, np.log(600.0))))
    Nk = int(np.exp(rng.uniform(0.0, np.log(9000.0))))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    splits = [0, 0, 2, 7, 16, 64][int(rng.integers(6))]
    bshd = bool(rng.integers(2))
    scale = float(np.float32(1.0 / np.sqrt(d))) if rng.random() < 0.6 else float(rng.uniform(-0.3, 0.4))
    hot = dtype != "f32" and rng.random() < 0.3
    return dict(dtype=dtype, d=d, N=N, Nk=Nk, B=B, H=H, splits=splits, bshd=bshd, scale=scale,
                hot=hot, seed=9500 + i)


def _random_id(i):
    c = _random_case(i)
    return (f"{i}-{c['dtype']}-d{c['d']}-N{c['N']}-Nk{c['Nk']}-B{c['B']}H{c['H']}-S{c['splits']}"
            f"{'-bshd' if c['bshd'] else ''}{'-hot' if c['hot'] else ''}")


@pytest.mark.parametrize("i", range(NRANDOM), ids=[_random_id(i) for i in range(NRANDOM)])
def test_cross_lengths_random(i):
    """A seeded sweep over dtype, head dim, N (log-uniform 1-600), Nk
    (log-uniform 1-9000), B, H, key splits, layout, scale and hot keys; the
    library picks the kernel (decode, pipelined or ping-pong)."""
    c = _random_case(i)
    _compare(c["dtype"], c["d"], c["B"], c["H"], c["N"], c["Nk"], c["seed"], scale=c["scale"],
             splits=c["splits"], bshd=c["bshd"], hot=c["hot"], what=_random_id(i))
