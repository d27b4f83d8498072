"""GPU parity over a seeded random sweep of shapes and options.

Each case draws, from its own seed: the dtype (bf16, fp16, fp32), the head
dimension, N (log-uniform from 16 to 3000 in four cases of five, else 1 to
15; most cases end in a ragged key tile), B and H, the causal flag, the layout (contiguous or the
[B, N, H, d] view), the scale (1/sqrt(d) or a random value of either sign),
optionally 1 % hot keys (x8), and for the 16-bit dtypes which kernel runs
(the library's own choice, or the ping-pong, pipelined or key-split
pipelined kernel forced).  Every element of O and lse is compared with the
fp64 oracle at the bars of test_parity.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from test_parity import check

pytestmark = pytest.mark.gpu

NCASES = 100


def case(i):
    rng = np.random.default_rng(7000 + i)
    dtype = ["bf16", "f16", "f32"][int(rng.integers(3))]
    d = [64, 128][int(rng.integers(2))]
    if rng.random() < 0.8:
        N = int(np.exp(rng.uniform(math.log(16.0), math.log(3000.0))))
    else:
        N = int(rng.integers(1, 16))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    causal = bool(rng.integers(2))
    bshd = bool(rng.integers(2))
    scale = 1.0 / math.sqrt(d) if rng.random() < 0.6 else float(rng.uniform(-0.3, 0.5))
    hot = dtype != "f32" and rng.random() < 0.25
    kernel = None
    if dtype != "f32":
        kernel = [None, "pingpong", "pipelined", "pipelined2"][int(rng.integers(4))]
    return dict(dtype=dtype, d=d, N=N, B=B, H=H, causal=causal, bshd=bshd, scale=scale, hot=hot,
                kernel=kernel, seed=7000 + i)


def _ident(i):
    c = case(i)
    return (f"{i}-{c['dtype']}-d{c['d']}-N{c['N']}-B{c['B']}H{c['H']}"
            f"{'-causal' if c['causal'] else ''}{'-bshd' if c['bshd'] else ''}"
            f"{'-hot' if c['hot'] else ''}-{c['kernel'] or 'auto'}")


@pytest.mark.parametrize("i", range(NCASES), ids=[_ident(i) for i in range(NCASES)])
def test_random_case(i, monkeypatch):
    import attention_attn_fwd_07_amd as attn
    c = case(i)
    if c["kernel"] is not None:
        monkeypatch.setenv("ATTN_FWD_KERNEL", c["kernel"])
    kw = dict(hot_frac=0.01, hot_mult=8.0) if c["hot"] else {}
    q, k, v = datagen.make_qkv(c["B"], c["H"], c["N"], c["d"], c["dtype"], seed=c["seed"], **kw)
    dev = torch.device("cuda:0")
    if c["bshd"]:
        # the same values held as [B, N, H, d] and viewed as [B, H, N, d]
        qd, kd, vd = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for t in (q, k, v))
    else:
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty(q.shape, dtype=qd.dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    attn.attn_fwd(qd, kd, vd, o, lse, c["scale"], causal=c["causal"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, c["scale"], causal=c["causal"])
    check(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, c["dtype"],
          _ident(i))
