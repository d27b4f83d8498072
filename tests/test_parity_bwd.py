"""GPU parity of the attention backward (include/attn_bwd.h) against the fp64
oracle's gradients (oracle.attention_backward).

The backward is fed the GPU forward's own O and lse, as a training step would
be, and its dQ, dK, dV are compared element by element with the exact
gradients of the definition at the same rounded inputs.

Tolerance, derived from the arithmetic (no figure is given for the backward):
the kernels round P and dS to the element type before their MFMA products
(relative error at most rr = 2^-8 for bf16, 2^-11 for fp16), accumulate in
fp32, take D = rowsum(dO * O) from the forward's rounded O, recompute P from
the forward's fp32 lse, and round each gradient to the element type.
Propagating each of these first-order errors through dS = P (dP - D),
dV = P^T dO, dQ = scale dS K and dK = scale dS^T Q with absolute values gives
a per-element bound (worst case: all rounding errors aligned); every element
must lie within 1.25x that bound (plus 1e-6).  fp32 accumulation is bounded
by gamma_n = n 2^-24 times the sum of absolute terms.

That worst case cannot see a small systematic bias, so each gradient's
relative Frobenius error is held as well, to a bar from the same roundings
taken as what they are on these inputs, independent and unbiased:
round-to-nearest-even leaves a relative error uniform in [-u, u] (u = 2^-8
for bf16, 2^-11 for fp16), RMS u / sqrt(3), and a gradient element collects
about three such roundings (P or dS before its product, the gradient itself
on output; the products' terms have random signs, so a rounding of the terms
moves the sum by the same relative RMS as it moves the terms), which gives a
relative RMS near u.  The bar is 2u: bf16 7.8e-3, fp16 9.8e-4.  A bias such
as a D off by a percent, or P taken from a wrong lse, exceeds it.

fp32 inputs (their own kernels, nothing rounded below fp32): u = 2^-24 in
the bound.  Their rel-F bar is set by what 2u leaves out: P is recomputed
from the forward's fp32 lse, which carries a few ulps of |lse| (about 1e-6
relative in P), and each product accumulates d or N fp32 terms (RMS near
sqrt(n) 2^-24, under 1e-6 here); the bar 1e-5 is five times their sum.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

RR = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}
RELF = {"bf16": 2.0 * RR["bf16"], "f16": 2.0 * RR["f16"], "f32": 1e-5}


def _attn():
    import attention_attn_fwd_07_amd as attn
    return attn


def gpu_fwd_bwd(q, k, v, g, scale, causal):
    attn = _attn()
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    o, lse = attn.fwd(qd, kd, vd, scale, causal=causal)
    dq, dk, dv = attn.bwd(qd, kd, vd, o, lse, gd, scale, causal=causal)
    torch.cuda.synchronize()
    return [t.cpu().double().numpy() for t in (o, lse, dq, dk, dv)]


def bounds(q, k, v, g, o_gpu, lse_gpu, scale, causal, dtype):
    """Per-element error bounds for dq, dk, dv (float64, see module doc)."""
    rr = RR[dtype]
    q, k, v, g = (t.double().numpy() for t in (q, k, v, g))
    B, H, N, d = q.shape
    gam_d, gam_n = d * 2.0 ** -24, max(N, d) * 2.0 ** -24
    _, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(q, k, v, g, scale, causal=causal)
    bq, bk, bv = (np.empty_like(x) for x in (q, k, v))
    a = abs(scale)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, gh = q[b, h], k[b, h], v[b, h], g[b, h]
            p = oracle.softmax_probs(qh, kh, scale, causal=causal)
            o = p @ vh
            dp = gh @ vh.T
            dd = (gh * o).sum(axis=1, keepdims=True)
            ds = p * (dp - dd)
            # errors of the kernels' inputs to dS
            e_lse = np.abs(lse_gpu[b, h] - lse_ref[b, h])[:, None] + 3e-7
            e_s = gam_d * a * (np.abs(qh) @ np.abs(kh).T)
            e_p = p * (e_lse + e_s)
            absgo = np.abs(gh) * np.abs(o_gpu[b, h])
            e_d = (rr + gam_d) * absgo.sum(axis=1, keepdims=True)
            e_d += np.abs((gh * (o_gpu[b, h] - o)).sum(axis=1, keepdims=True))
            e_dp = gam_d * (np.abs(gh) @ np.abs(vh).T)
            e_ds = e_p * np.abs(dp - dd) + p * (e_dp + e_d)
            e_ds += rr * (np.abs(ds) + e_ds)           # dS rounded for the MFMA
            bv[b, h] = ((e_p + rr * p).T @ np.abs(gh) + gam_n * (p.T @ np.abs(gh))
                        + rr * np.abs(dv_ref[b, h]))
            bq[b, h] = (a * (e_ds @ np.abs(kh)) + gam_n * a * (np.abs(ds) @ np.abs(kh))
                        + rr * np.abs(dq_ref[b, h]))
            bk[b, h] = (a * (e_ds.T @ np.abs(qh)) + gam_n * a * (np.abs(ds).T @ np.abs(qh))
                        + rr * np.abs(dk_ref[b, h]))
    return (dq_ref, dk_ref, dv_ref), (bq, bk, bv)


def check_grads(q, k, v, g, scale, causal, dtype, what):
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, g, scale, causal)
    refs, bnds = bounds(q, k, v, g, o, lse, scale, causal, dtype)
    for name, got, ref, bnd in zip(("dq", "dk", "dv"), (dq, dk, dv), refs, bnds):
        assert np.all(np.isfinite(got)), f"{what}: {name} not finite"
        err = np.abs(got - ref)
        ratio = float((err / (1.25 * bnd + 1e-6)).max())
        ref_norm = np.linalg.norm(ref)
        relf = float(np.linalg.norm(got - ref) / max(ref_norm, 1e-30))
        assert ratio <= 1.0, (f"{what}: {name} error exceeds its bound (ratio {ratio:.2f}, "
                              f"rel-F {relf:.2e})")
        # rel-F is meaningful only where the gradient is not zero in exact
        # arithmetic (N = 1 gives dQ = dK = 0: there only the bound applies)
        if ref_norm > 1e-6 * math.sqrt(ref.size):
            assert relf <= RELF[dtype], f"{what}: {name} rel-F {relf:.2e} > {RELF[dtype]:.2e}"
    return dq, dk, dv


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 300, 640])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_shapes(dtype, d, N, causal):
    q, k, v = datagen.make_qkv(1, 2, N, d, dtype, seed=700 + N + d)
    g = datagen.make_grad(1, 2, N, d, dtype, seed=700 + N + d)
    check_grads(q, k, v, g, 1.0 / math.sqrt(d), causal, dtype,
                f"bwd {dtype} d={d} N={N} causal={causal}")


@pytest.mark.parametrize("scale", [-0.125, 0.02, 0.5])
def test_bwd_scales_and_hot_keys(scale):
    q, k, v = datagen.make_qkv(1, 2, 500, 64, "bf16", seed=71, hot_frac=0.01, hot_mult=8.0)
    g = datagen.make_grad(1, 2, 500, 64, "bf16", seed=71)
    check_grads(q, k, v, g, scale, False, "bf16", f"bwd hot keys scale {scale}")


def test_bwd_larger_causal_and_deterministic():
    q, k, v = datagen.make_qkv(2, 3, 1024, 128, "bf16", seed=72)
    g = datagen.make_grad(2, 3, 1024, 128, "bf16", seed=72)
    dq, dk, dv = check_grads(q, k, v, g, 1 / math.sqrt(128), True, "bf16", "bwd B2 H3 N1024")
    _, _, dq2, dk2, dv2 = gpu_fwd_bwd(q, k, v, g, 1 / math.sqrt(128), True)
    assert np.array_equal(dq, dq2) and np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_bwd_closed_forms_at_size():
    """B=2 H=16 N=4096 d=128 bf16 (the forward's 4096-length shape): the keys'
    dK sum to zero and the keys' dV sum to the queries' dO, up to the same
    error bounds summed over keys (checked on four heads)."""
    q, k, v = datagen.make_qkv(2, 16, 4096, 128, "bf16", seed=3)
    g = datagen.make_grad(2, 16, 4096, 128, "bf16", seed=3)
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, g, 1 / math.sqrt(128), False)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    heads = [(0, 0), (0, 7), (1, 3), (1, 15)]
    qs, ks, vs, gs = (t[[b for b, _ in heads], [h for _, h in heads]][:, None]
                      for t in (q, k, v, g))
    os_ = o[[b for b, _ in heads], [h for _, h in heads]][:, None]
    ls = lse[[b for b, _ in heads], [h for _, h in heads]][:, None]
    refs, bnds = bounds(qs, ks, vs, gs, os_, ls, 1 / math.sqrt(128), False, "bf16")
    for i, (b, h) in enumerate(heads):
        for got, ref, bnd in zip((dq[b, h], dk[b, h], dv[b, h]), refs, bnds):
            assert np.all(np.abs(got - ref[i, 0]) <= 1.25 * bnd[i, 0] + 1e-6)
    sum_bound = 1.25 * bnds[1].sum(axis=2) + 1e-4
    assert np.all(np.abs(dk[[b for b, _ in heads], [h for _, h in heads]].sum(axis=1))
                  <= sum_bound[:, 0])


def test_bwd_binding_rejects_mixed_dtypes_and_missing_lse():
    attn = _attn()
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        attn.bwd(q, q.bfloat16(), q, q, torch.zeros(1, 1, 64, device="cuda"), q)
    qb = q.bfloat16()
    with pytest.raises(ValueError):
        attn.bwd(qb, qb, qb, qb, None, qb)


@pytest.mark.parametrize("causal", [False, True])
def test_autograd_wrapper(causal):
    """attention() as a torch op: O equals fwd's, the gradients equal the
    direct attn_bwd call's (the same kernels on the same saved tensors), and
    those hold the oracle's bounds."""
    attn = _attn()
    q, k, v = datagen.make_qkv(1, 2, 300, 64, "bf16", seed=811)
    g = datagen.make_qkv(1, 2, 300, 64, "bf16", seed=812)[0]
    scale = 0.125
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev).requires_grad_(True) for t in (q, k, v))
    o = attn.attention(qd, kd, vd, scale, causal=causal)
    o.backward(g.to(dev))
    o_ref, lse_ref = attn.fwd(qd.detach(), kd.detach(), vd.detach(), scale, causal=causal)
    grads = attn.bwd(qd.detach(), kd.detach(), vd.detach(), o_ref, lse_ref, g.to(dev), scale,
                     causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for got, want in zip((qd.grad, kd.grad, vd.grad), grads):
        assert torch.equal(got, want)
    check_grads(q, k, v, g, scale, causal, "bf16", f"autograd causal={causal}")


def _bwd_case(i):
    rng = np.random.default_rng(9100 + i)
    dtype = ["bf16", "f16"][int(rng.integers(2))]
    d = [64, 128][int(rng.integers(2))]
    N = int(np.exp(rng.uniform(0.0, math.log(1200.0))))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    causal = bool(rng.integers(2))
    scale = 1.0 / math.sqrt(d) if rng.random() < 0.6 else float(rng.uniform(-0.3, 0.4))
    return dtype, d, N, B, H, causal, scale, 9100 + i


@pytest.mark.parametrize("i", range(24), ids=lambda i: "{}-{}-d{}-N{}-B{}H{}-{}".format(
    i, *_bwd_case(i)[:5], "causal" if _bwd_case(i)[5] else "plain"))
def test_bwd_random_case(i):
    """A seeded random sweep (dtype, head dim, N, B, H, causal, scale): every
    gradient element within its derived bound, rel-F within 2u."""
    dtype, d, N, B, H, causal, scale, seed = _bwd_case(i)
    q, k, v = datagen.make_qkv(B, H, N, d, dtype, seed=seed)
    g = datagen.make_qkv(B, H, N, d, dtype, seed=seed + 50000)[0]
    check_grads(q, k, v, g, scale, causal, dtype, f"random bwd case {i}")


def _bwd_case32(i):
    rng = np.random.default_rng(9300 + i)
    d = [64, 128][int(rng.integers(2))]
    N = int(np.exp(rng.uniform(0.0, math.log(700.0))))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    causal = bool(rng.integers(2))
    scale = 1.0 / math.sqrt(d) if rng.random() < 0.6 else float(rng.uniform(-0.3, 0.4))
    return d, N, B, H, causal, scale, 9300 + i


@pytest.mark.parametrize("i", range(12), ids=lambda i: "{}-d{}-N{}-B{}H{}-{}".format(
    i, *_bwd_case32(i)[:4], "causal" if _bwd_case32(i)[4] else "plain"))
def test_bwd_f32_random_case(i):
    """fp32 inputs: a seeded sweep of head dim, N, B, H, causal and scale,
    every gradient element within its bound, rel-F within 1e-5."""
    d, N, B, H, causal, scale, seed = _bwd_case32(i)
    q, k, v = datagen.make_qkv(B, H, N, d, "f32", seed=seed)
    g = datagen.make_qkv(B, H, N, d, "f32", seed=seed + 50000)[0]
    check_grads(q, k, v, g, scale, causal, "f32", f"random fp32 bwd case {i}")


def test_autograd_wrapper_f32():
    """attention() on fp32 tensors: gradients from the fp32 backward."""
    attn = _attn()
    q, k, v = datagen.make_qkv(1, 2, 150, 128, "f32", seed=813)
    g = datagen.make_grad(1, 2, 150, 128, "f32", seed=813)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev).requires_grad_(True) for t in (q, k, v))
    o = attn.attention(qd, kd, vd, 0.1, causal=True)
    o.backward(g.to(dev))
    torch.cuda.synchronize()
    o_ref, _ = oracle.attention(q, k, v, 0.1, causal=True)
    assert np.abs(o.detach().cpu().double().numpy() - o_ref).max() <= 1e-4
    refs = oracle.attention_backward(q, k, v, g, 0.1, causal=True)
    for got, ref in zip((qd.grad, kd.grad, vd.grad), refs):
        got = got.cpu().double().numpy()
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-5
