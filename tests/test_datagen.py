"""The seeded input generator: deterministic, right shapes/dtypes, right recipe."""
import math

import numpy as np
import torch

import datagen


def test_deterministic_and_seed_sensitive():
    a = datagen.make_qkv(2, 3, 17, 64, "bf16", seed=5)
    b = datagen.make_qkv(2, 3, 17, 64, "bf16", seed=5)
    c = datagen.make_qkv(2, 3, 17, 64, "bf16", seed=6)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert not torch.equal(a[0].float(), c[0].float())


def test_shapes_dtypes_contiguity():
    for dt, tdt in (("f32", torch.float32), ("f16", torch.float16), ("bf16", torch.bfloat16)):
        q, k, v = datagen.make_qkv(1, 2, 33, 128, dt, seed=1)
        for t in (q, k, v):
            assert t.shape == (1, 2, 33, 128) and t.dtype == tdt and t.is_contiguous()
            assert t.device.type == "cpu"


def test_values_are_the_rounded_normal_draws():
    q, k, v = datagen.make_qkv(1, 1, 8, 64, "f32", seed=3, mult=0.5)
    rng = np.random.Generator(np.random.PCG64(3))
    qq = rng.standard_normal((1, 1, 8, 64)) * 0.5
    kk = rng.standard_normal((1, 1, 8, 64)) * 0.5
    vv = rng.standard_normal((1, 1, 8, 64)) * 0.5
    assert np.array_equal(q.numpy(), qq.astype(np.float32))
    assert np.array_equal(k.numpy(), kk.astype(np.float32))
    assert np.array_equal(v.numpy(), vv.astype(np.float32))


def test_hot_keys_exact_count_and_factor():
    B, H, N, d = 1, 3, 1000, 64
    q, k, v = datagen.make_qkv(B, H, N, d, "f32", seed=9, hot_frac=0.01, hot_mult=8.0)
    _, k_plain, _ = datagen.make_qkv(B, H, N, d, "f32", seed=9)
    idx = datagen.hot_key_indices(B, H, N, d, seed=9, hot_frac=0.01)
    for h in range(H):
        hot = idx[(0, h)]
        assert len(hot) == 10 and len(np.unique(hot)) == 10
        ratio_rows = np.flatnonzero(~np.all(k[0, h].numpy() == k_plain[0, h].numpy(), axis=1))
        assert np.array_equal(np.sort(ratio_rows), hot)
        np.testing.assert_array_equal(k[0, h, hot].numpy(), 8.0 * k_plain[0, h, hot].numpy())


def test_workload_table():
    w = datagen.WORKLOADS
    assert [(x.B, x.H, x.N, x.d, x.dtype) for x in w.values()] == [
        (1, 1, 128, 64, "f32"), (4, 8, 1024, 64, "bf16"), (2, 16, 4096, 128, "bf16"),
        (1, 32, 16384, 128, "f16"), (1, 8, 65536, 64, "bf16")]
    assert w[4].mult == 0.5 and w[5].hot_keys == 655
    assert w[3].scale == float(np.float32(1 / math.sqrt(128)))
    assert w[3].flops == 4 * 2 * 16 * 4096 ** 2 * 128


def test_make_grad_is_seeded_and_independent_of_qkv():
    g1 = datagen.make_grad(1, 2, 33, 64, "bf16", seed=5)
    g2 = datagen.make_grad(1, 2, 33, 64, "bf16", seed=5)
    q, k, v = datagen.make_qkv(1, 2, 33, 64, "bf16", seed=5)
    assert torch.equal(g1, g2) and g1.dtype == torch.bfloat16 and g1.is_contiguous()
    assert not torch.equal(g1, q) and not torch.equal(g1, v)


def test_make_qkv_kv_shapes_and_self_attention_case():
    q, k, v = datagen.make_qkv_kv(2, 3, 5, 70, 64, "bf16", seed=8, hot_frac=0.1, hot_mult=8.0)
    assert q.shape == (2, 3, 5, 64) and k.shape == v.shape == (2, 3, 70, 64)
    # with Nk = N the values are exactly those of make_qkv
    a = datagen.make_qkv(2, 3, 40, 64, "f16", seed=8, hot_frac=0.05, hot_mult=8.0)
    b = datagen.make_qkv_kv(2, 3, 40, 40, 64, "f16", seed=8, hot_frac=0.05, hot_mult=8.0)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    # hot keys are counted from the key length: 7 of 70 rows per head are x8
    _, kp, _ = datagen.make_qkv_kv(2, 3, 5, 70, 64, "f32", seed=8)
    _, kh, _ = datagen.make_qkv_kv(2, 3, 5, 70, 64, "f32", seed=8, hot_frac=0.1, hot_mult=8.0)
    changed = (~np.all(kh.numpy() == kp.numpy(), axis=-1)).sum(axis=-1)
    assert np.all(changed == 7)
