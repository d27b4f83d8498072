"""GPU parity of attn_fwd_ex: the causal variant and strided layouts.

Causal: query row i attends keys 0..i (page 1 section 4's note on the causal
mask; page 3 section 3's decoder layer masks future positions before the
softmax, section 6's wrapper passes the flag).  Compared element by element
with the fp64 oracle's causal definition at the same bars as the plain path.

Strides: the same tensors presented as [B, N, H, d] views, as padded rows and
as mixtures give results bit-identical to the contiguous call (same kernel,
same arithmetic, only the addressing differs), and match the oracle.
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


def run(q, k, v, scale, causal=False, o=None):
    attn = _attn()
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if o is None:
        o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    attn.attn_fwd(q, k, v, o, lse, scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


def causal_parity(q, k, v, scale, dtype, what):
    dev = torch.device("cuda:0")
    o, lse = run(q.to(dev), k.to(dev), v.to(dev), scale, causal=True)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=True)
    check(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, dtype, what)
    return o, lse


# ---------------------------------------------------------------------------
# causal
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", ["pingpong", "pipelined"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("bf16", 64), ("f16", 128)])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 200, 256, 257, 600])
def test_causal_16bit(kernel, dtype, d, N, monkeypatch):
    monkeypatch.setenv("ATTN_FWD_KERNEL", kernel)
    q, k, v = datagen.make_qkv(1, 3, N, d, dtype, seed=300 + N + d)
    causal_parity(q, k, v, 1.0 / math.sqrt(d), dtype, f"causal {kernel} {dtype} d={d} N={N}")


@pytest.mark.parametrize("kernel", ["pingpong", "pipelined"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("N", [1000, 2100])
def test_causal_long_rows(kernel, dtype, d, N, monkeypatch):
    """Rows long enough that the waves of a 256-row block run a stretch of
    tiles they see whole before the tiles that cross their diagonal (the
    ping-pong kernel takes the two stretches in separate loops), over several
    query blocks per head and a ragged last block."""
    monkeypatch.setenv("ATTN_FWD_KERNEL", kernel)
    q, k, v = datagen.make_qkv(1, 2, N, d, dtype, seed=310 + N + d)
    causal_parity(q, k, v, 1.0 / math.sqrt(d), dtype, f"causal long {kernel} {dtype} d={d} N={N}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 31, 33, 128, 129, 300])
def test_causal_f32(d, N):
    q, k, v = datagen.make_qkv(2, 2, N, d, "f32", seed=400 + N + d)
    causal_parity(q, k, v, 1.0 / math.sqrt(d), "f32", f"causal f32 d={d} N={N}")


def test_causal_large_grid():
    """B=2 H=16 N=4096 d=128 bf16: the ping-pong kernel's grid, every head whole."""
    q, k, v = datagen.make_qkv(2, 16, 4096, 128, "bf16", seed=3)
    causal_parity(q, k, v, 1.0 / math.sqrt(128), "bf16", "causal B2 H16 N4096 d128")


@pytest.mark.parametrize("kernel", ["pingpong", "pipelined"])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_hot_keys_and_negative_scale(kernel, d, monkeypatch):
    monkeypatch.setenv("ATTN_FWD_KERNEL", kernel)
    q, k, v = datagen.make_qkv(1, 2, 1500, d, "bf16", seed=57, hot_frac=0.01, hot_mult=8.0)
    causal_parity(q, k, v, 0.125, "bf16", f"causal hot keys {kernel} d={d}")
    causal_parity(q, k, v, -0.125, "bf16", f"causal negative scale {kernel} d={d}")


@pytest.mark.parametrize("kernel", ["pingpong", "pipelined"])
def test_causal_first_row_is_v0(kernel, monkeypatch):
    """Row 0 sees key 0 only: P = 2^0 = 1 exactly, so O[0] = V[0] bit for bit."""
    monkeypatch.setenv("ATTN_FWD_KERNEL", kernel)
    q, k, v = datagen.make_qkv(2, 2, 333, 128, "bf16", seed=58)
    dev = torch.device("cuda:0")
    o, lse = run(q.to(dev), k.to(dev), v.to(dev), 0.1, causal=True)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
    s00 = 0.1 * (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1)
    assert torch.allclose(lse[:, :, 0].cpu().double(), s00, atol=1e-5, rtol=0)


def test_causal_deterministic_and_last_row_matches_plain():
    """The last query row sees every key: it equals the non-causal result."""
    q, k, v = datagen.make_qkv(1, 4, 1000, 128, "bf16", seed=59)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o1, l1 = run(qd, kd, vd, 0.09, causal=True)
    o2, l2 = run(qd, kd, vd, 0.09, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = run(qd, kd, vd, 0.09, causal=False)
    o_ref, lse_ref = oracle.attention(q, k, v, 0.09)
    last = o1[:, :, -1].cpu().double().numpy()
    assert np.abs(last - o_ref[:, :, -1]).max() <= TOL["bf16"]["maxabs"]


# ---------------------------------------------------------------------------
# strided layouts
# ---------------------------------------------------------------------------

def bshd(t):
    """The same values held as a [B, N, H, d] buffer, viewed as [B, H, N, d]."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def padded(t, pad):
    """The same values in rows of d + pad elements (a slice of a wider buffer)."""
    B, H, N, d = t.shape
    buf = torch.full((B, H, N, d + pad), float("nan"), dtype=t.dtype, device=t.device)
    buf[..., :d] = t
    return buf[..., :d]


@pytest.mark.parametrize("kernel", ["pingpong", "pipelined", "pipelined2"])
@pytest.mark.parametrize("dtype,d,N", [("bf16", 128, 1000), ("f16", 64, 513), ("bf16", 64, 64),
                                       ("f32", 64, 300), ("f32", 128, 77)])
@pytest.mark.parametrize("causal", [False, True])
def test_strided_bit_identical_to_contiguous(kernel, dtype, d, N, causal, monkeypatch):
    monkeypatch.setenv("ATTN_FWD_KERNEL", kernel)
    q, k, v = datagen.make_qkv(2, 3, N, d, dtype, seed=500 + N)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o_ref, l_ref = run(qd, kd, vd, 0.11, causal)
    for what, (qq, kk, vv) in {
        "bshd all": (bshd(qd), bshd(kd), bshd(vd)),
        "padded rows": (padded(qd, 8), padded(kd, 64), padded(vd, 24)),
        "mixed": (bshd(qd), kd, padded(vd, 40)),
    }.items():
        assert not qq.is_contiguous() or what == "mixed"
        o, lse = run(qq, kk, vv, 0.11, causal)
        assert torch.equal(o.view(torch.int16) if dtype != "f32" else o,
                           o_ref.view(torch.int16) if dtype != "f32" else o_ref), what
        assert torch.equal(lse, l_ref), what
    # strided output: O written into a [B, N, H, d] buffer
    obuf = torch.empty(2, N, 3, d, dtype=qd.dtype, device=dev)
    o, lse = run(bshd(qd), bshd(kd), bshd(vd), 0.11, causal, o=obuf.transpose(1, 2))
    assert torch.equal(obuf.transpose(1, 2), o_ref)
    o64, lref = oracle.attention(q, k, v, 0.11, causal=causal)
    check(obuf.transpose(1, 2).cpu().double().numpy(), lse.cpu().double().numpy(), o64, lref,
          dtype, f"strided {kernel} {dtype} d={d} N={N} causal={causal}")


def test_strided_large_grid_bshd():
    """B=2 H=16 N=4096 d=128 bf16 in [B, N, H, d] layout (ping-pong kernel's grid)."""
    q, k, v = datagen.workload_inputs(3)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o_ref, l_ref = run(qd, kd, vd, 1 / math.sqrt(128))
    o, lse = run(bshd(qd), bshd(kd), bshd(vd), 1 / math.sqrt(128))
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_binding_rejects_bad_strides():
    attn = _attn()
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # head dim not contiguous
        attn.fwd(torch.zeros(1, 2, 64, 16, dtype=torch.bfloat16, device="cuda").transpose(2, 3),
                 q, q)
    buf = torch.zeros(1, 2, 16, 68, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # row stride 68 is not a multiple of 8
        attn.fwd(buf[..., :64], q, q)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f16", 128), ("f32", 64)])
def test_broadcast_key_row_gives_mean_of_v(dtype, d):
    """K as one row broadcast over every (b, h, n) (all leading strides 0, the
    form ``expand`` makes): every score of a row is equal, so O is the mean of
    V's rows and lse = scale q.k0 + ln N (page 3 section 3's softmax of equal
    scores).  The binding copies such an input to a contiguous tensor; the
    result matches the oracle on the materialised keys."""
    B, H, N = 2, 3, 300
    q, k, v = datagen.make_qkv(B, H, N, d, dtype, seed=400 + d)
    dev = torch.device("cuda:0")
    k0 = k[:1, :1, :1].to(dev)
    kb = k0.expand(B, H, N, d)
    assert not kb.is_contiguous() and tuple(kb.stride()[:3]) == (0, 0, 0)
    scale = 1.0 / math.sqrt(d)
    o, lse = run(q.to(dev), kb, v.to(dev), scale)
    o64 = o.cpu().double().numpy()
    v64 = v.double().numpy()
    tol = TOL[dtype]
    assert np.abs(o64 - v64.mean(axis=2, keepdims=True)).max() <= tol["maxabs"]
    k_full = k[:1, :1, :1].expand(B, H, N, d).contiguous()
    o_ref, lse_ref = oracle.attention(q, k_full, v, scale)
    check(o64, lse.cpu().double().numpy(), o_ref, lse_ref, dtype, f"broadcast k {dtype} d={d}")


def test_broadcast_output_is_rejected():
    attn = _attn()
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros(1, 1, 1, 64, dtype=torch.bfloat16, device="cuda").expand(1, 2, 16, 64)
    with pytest.raises(ValueError):
        attn.attn_fwd(q, q.clone(), q.clone(), o, None, 0.125)
