"""Pins for the fp64 oracle, checked against things other than itself.

Each pin is a function of an ``attn(q, k, v, scale) -> (o, lse)`` callable so
that the same pins can be run against deliberately broken copies of the oracle
(``test_planted_mistakes_are_caught``): a dropped term, a wrong sign, a wrong
axis, a transposed operand or an off-by-one must each fail at least one pin.

What pins what:

* hand-worked fixtures (``tests/golden/hand_worked.json``): every step, on
  values derived by hand from the definition;
* brute force: pure-Python ``math.exp``/``math.fsum`` loops of the textbook
  softmax (no max subtraction) on tiny shapes;
* library special case: ``torch.nn.functional.scaled_dot_product_attention``
  in float64 on the CPU (the same definition, someone else's code);
* closed forms: softmax rows sum to one, identical keys give the mean of V,
  constant V gives that constant, scale 0 gives mean(V) and lse = ln N, N = 1
  gives v_0 and lse = scale * q.k_0, one dominant key gives its value row;
* invariants: joint permutation of K/V rows, a common shift of all K rows
  (O unchanged, lse shifted by scale * q.u), linearity in V, and
  max_j s_ij <= lse_i <= max_j s_ij + ln N;
* the method's own claim: the one-pass online recurrence (page 1 section 4,
  page 3 section 5) equals the two-pass definition for several block sizes,
  including block sizes that do not divide N.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import definition as attention_mod
from oracle.online import attention_online

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
RNG = np.random.default_rng(20261202)


def _attn(q, k, v, scale):
    return oracle.attention(q, k, v, scale, workers=1)


def _rand(B, H, N, d, seed, scale=1.0, dv=None):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, N, d)) * scale
    k = r.standard_normal((B, H, N, d)) * scale
    v = r.standard_normal((B, H, N, d if dv is None else dv))
    return q, k, v


# --------------------------------------------------------------------------
# pins, each a function of an attention callable
# --------------------------------------------------------------------------

def pin_golden(attn):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"])[None, None]
        k = np.array(c["k"])[None, None]
        v = np.array(c["v"])[None, None]
        o, lse = attn(q, k, v, c["scale"])
        np.testing.assert_allclose(o[0, 0], np.array(c["o"]), rtol=1e-13, atol=1e-13,
                                   err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0], np.array(c["lse"]), rtol=1e-13, atol=1e-13,
                                   err_msg=c["name"])


def _brute_row(qi, K, V, scale):
    """Textbook softmax attention of one query row: no max subtraction."""
    s = [scale * math.fsum(a * b for a, b in zip(qi, kj)) for kj in K]
    e = [math.exp(x) for x in s]
    l = math.fsum(e)
    o = [math.fsum(e[j] * V[j][c] for j in range(len(K))) / l for c in range(len(V[0]))]
    return o, math.log(l)


def pin_brute_force(attn):
    for (N, d, seed) in [(1, 1, 0), (2, 4, 1), (3, 8, 2), (5, 4, 3), (17, 8, 4), (17, 1, 5)]:
        q, k, v = _rand(1, 2, N, d, seed)
        scale = 0.7
        o, lse = attn(q, k, v, scale)
        for h in range(2):
            Q, K, V = q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist()
            for i in range(N):
                ob, lb = _brute_row(Q[i], K, V, scale)
                np.testing.assert_allclose(o[0, h, i], ob, rtol=1e-12, atol=1e-12)
                assert abs(lse[0, h, i] - lb) <= 1e-12 * max(1.0, abs(lb))


def pin_sdpa(attn):
    for (B, H, N, d, seed, scale) in [(2, 3, 33, 16, 7, 0.25), (1, 2, 70, 64, 8, 0.125),
                                      (1, 1, 9, 5, 9, -0.6)]:
        q, k, v = _rand(B, H, N, d, seed)
        o, lse = attn(q, k, v, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        ref_lse = torch.logsumexp(scale * (tq @ tk.transpose(-1, -2)), dim=-1)
        np.testing.assert_allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def pin_rows_sum_to_one(attn):
    # With V = I (d_v = N) the output rows are the attention weights themselves.
    N = 23
    q, k, _ = _rand(1, 1, N, 6, 11)
    v = np.eye(N)[None, None]
    o, _ = attn(q, k, v, 0.9)
    assert np.all(o >= 0.0)
    np.testing.assert_allclose(o.sum(axis=-1), 1.0, atol=1e-12)
    # the weights are those of the definition
    np.testing.assert_allclose(o[0, 0], oracle.softmax_probs(q[0, 0], k[0, 0], 0.9), atol=1e-13)


def pin_identical_keys(attn):
    N, d = 19, 8
    q, _, v = _rand(1, 2, N, d, 12)
    k = np.broadcast_to(RNG.standard_normal(d), (1, 2, N, d)).copy()
    o, lse = attn(q, k, v, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape),
                               atol=1e-13)
    s0 = 0.5 * (q @ k[..., :1, :].swapaxes(-1, -2))[..., 0]
    np.testing.assert_allclose(lse, s0 + math.log(N), atol=1e-12)


def pin_constant_v(attn):
    N, d = 21, 4
    q, k, _ = _rand(1, 1, N, d, 13, scale=2.0)
    c = np.array([1.5, -2.0, 0.25, 7.0])
    v = np.broadcast_to(c, (1, 1, N, d)).copy()
    o, _ = attn(q, k, v, 1.0)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=1e-13, atol=1e-13)


def pin_scale_zero(attn):
    N = 13
    q, k, v = _rand(2, 1, N, 3, 14)
    o, lse = attn(q, k, v, 0.0)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape),
                               atol=1e-13)
    np.testing.assert_allclose(lse, math.log(N), atol=1e-13)


def pin_single_key(attn):
    q, k, v = _rand(3, 2, 1, 7, 15)
    o, lse = attn(q, k, v, 0.3)
    np.testing.assert_allclose(o, v, atol=1e-14)
    np.testing.assert_allclose(lse, 0.3 * (q * k).sum(-1), atol=1e-13)


def pin_dominant_key(attn):
    # key 5 beats every other by a score gap >= 50: e^-50 ~ 2e-22 -> O = v_5.
    N, d = 12, 4
    q = np.zeros((1, 1, 3, d))
    q[..., 0] = [1.0, 2.0, 60.0]
    k = np.zeros((1, 1, N, d))
    k[0, 0, :, 0] = 0.1 * np.arange(N)
    k[0, 0, 5, 0] = 1000.0
    v = RNG.standard_normal((1, 1, N, d))
    qq = np.concatenate([q, np.zeros((1, 1, N - 3, d))], axis=2)  # square: same N
    o, lse = attn(qq, k, v, 1.0)
    for i, qi in enumerate([1.0, 2.0, 60.0]):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, 5], rtol=1e-13, atol=1e-13)
        assert abs(lse[0, 0, i] - 1000.0 * qi) <= 1e-12 * 1000.0 * qi


def pin_invariances(attn):
    N, d = 29, 8
    q, k, v = _rand(1, 1, N, d, 16)
    scale = 0.4
    o, lse = attn(q, k, v, scale)
    perm = RNG.permutation(N)
    o2, lse2 = attn(q, k[..., perm, :], v[..., perm, :], scale)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)
    u = RNG.standard_normal(d)
    o3, lse3 = attn(q, k + u, v, scale)
    np.testing.assert_allclose(o3, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse3, lse + scale * (q[0, 0] @ u), atol=1e-12)
    w = RNG.standard_normal((1, 1, N, d))
    ov, _ = attn(q, k, v, scale)
    ow, _ = attn(q, k, w, scale)
    ovw, _ = attn(q, k, 2.0 * v - 3.0 * w, scale)
    np.testing.assert_allclose(ovw, 2.0 * ov - 3.0 * ow, atol=1e-12)
    # lse is bounded by the row max and the row max plus ln N
    s = scale * (q[0, 0] @ k[0, 0].T)
    smax = s.max(axis=1)
    assert np.all(lse[0, 0] >= smax - 1e-12)
    assert np.all(lse[0, 0] <= smax + math.log(N) + 1e-12)
    # a query row attends to key rows of its own (b, h) only
    qb, kb, vb = _rand(2, 3, 10, 4, 17)
    ob, _ = attn(qb, kb, vb, 0.5)
    for b in range(2):
        for h in range(3):
            oh, _ = attn(qb[b:b + 1, h:h + 1], kb[b:b + 1, h:h + 1], vb[b:b + 1, h:h + 1], 0.5)
            np.testing.assert_allclose(ob[b, h], oh[0, 0], atol=1e-14)


def pin_online_matches(attn):
    for (N, bn) in [(50, 1), (50, 7), (64, 64), (130, 64), (130, 128), (33, 33)]:
        q, k, v = _rand(1, 2, N, 8, 100 + N + bn)
        k[..., ::9, :] *= 8.0  # a few hot keys move the running max late
        o, lse = attn(q, k, v, 0.6)
        o2, lse2 = attention_online(q, k, v, 0.6, bn)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-12)
    for (N, Nk, bn) in [(1, 130, 64), (7, 50, 16), (40, 9, 4)]:  # key length of its own
        r = np.random.default_rng(200 + N)
        q, k, v = (r.standard_normal((1, 2, n, 8)) for n in (N, Nk, Nk))
        k[..., ::9, :] *= 8.0
        o, lse = attn(q, k, v, 0.6)
        o2, lse2 = attention_online(q, k, v, 0.6, bn)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-12)


# --- query and key lengths that differ (N queries against Nk keys) --------

def _rand_kv(B, H, N, Nk, d, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, H, N, d)), r.standard_normal((B, H, Nk, d)),
            r.standard_normal((B, H, Nk, d)))


def pin_cross_brute_force(attn):
    """Pure-Python textbook softmax of every row, over all Nk keys."""
    for (N, Nk, d, seed) in [(1, 1, 4, 30), (1, 7, 4, 31), (3, 17, 8, 32), (17, 3, 8, 33),
                             (2, 40, 1, 34)]:
        q, k, v = _rand_kv(1, 2, N, Nk, d, seed)
        o, lse = attn(q, k, v, 0.8)
        assert o.shape == (1, 2, N, d) and lse.shape == (1, 2, N)
        for h in range(2):
            K, V = k[0, h].tolist(), v[0, h].tolist()
            for i in range(N):
                ob, lb = _brute_row(q[0, h, i].tolist(), K, V, 0.8)
                np.testing.assert_allclose(o[0, h, i], ob, rtol=1e-12, atol=1e-12)
                assert abs(lse[0, h, i] - lb) <= 1e-12 * max(1.0, abs(lb))


def pin_cross_sdpa(attn):
    """torch's SDPA in float64 with different query and key lengths."""
    for (B, H, N, Nk, d, seed, scale) in [(2, 3, 1, 90, 16, 35, 0.25), (1, 2, 70, 9, 64, 36, 0.125),
                                          (1, 1, 5, 130, 8, 37, -0.5)]:
        q, k, v = _rand_kv(B, H, N, Nk, d, seed)
        o, lse = attn(q, k, v, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        ref_lse = torch.logsumexp(scale * (tq @ tk.transpose(-1, -2)), dim=-1)
        np.testing.assert_allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def pin_cross_closed_forms(attn):
    """One query against Nk keys: scale 0 gives mean(V) over the Nk keys and
    lse = ln Nk; identical keys give the same mean; rows are those of the
    self-attention result over Nk queries whose first rows are these queries
    (query rows are independent), tying the cross case to the square one."""
    N, Nk, d = 3, 41, 8
    q, k, v = _rand_kv(2, 1, N, Nk, d, 38)
    mean_v = v.mean(axis=2, keepdims=True)
    o, lse = attn(q, k, v, 0.0)
    np.testing.assert_allclose(o, np.broadcast_to(mean_v, o.shape), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(Nk), atol=1e-13)
    same = np.broadcast_to(k[:, :, :1], k.shape).copy()
    o, lse = attn(q, same, v, 0.7)
    np.testing.assert_allclose(o, np.broadcast_to(mean_v, o.shape), atol=1e-13)
    s0 = 0.7 * (q @ same[:, :, :1].swapaxes(-1, -2))[..., 0]
    np.testing.assert_allclose(lse, s0 + math.log(Nk), atol=1e-12)
    full = np.concatenate([q, np.random.default_rng(39).standard_normal((2, 1, Nk - N, d))],
                          axis=2)
    o, lse = attn(q, k, v, 0.6)
    of, lf = attn(full, k, v, 0.6)
    np.testing.assert_allclose(o, of[:, :, :N], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lf[:, :, :N], rtol=1e-14, atol=1e-14)


PINS = [pin_golden, pin_brute_force, pin_sdpa, pin_rows_sum_to_one, pin_identical_keys,
        pin_constant_v, pin_scale_zero, pin_single_key, pin_dominant_key, pin_invariances,
        pin_online_matches, pin_cross_brute_force, pin_cross_sdpa, pin_cross_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_attn)


def test_chunked_and_threaded_is_identical():
    """Row chunking and the thread pool change values only by BLAS rounding order."""
    q, k, v = _rand(2, 3, 300, 16, 21)
    o1, l1 = oracle.attention(q, k, v, 0.25, workers=1, row_chunk=1000)
    o2, l2 = oracle.attention(q, k, v, 0.25, workers=4, row_chunk=37)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14, atol=1e-14)


def test_attention_rows_matches_full():
    q, k, v = _rand(2, 2, 90, 8, 22)
    o, lse = oracle.attention(q, k, v, 0.5, workers=1)
    idx = np.array([[0, 0, 0], [1, 1, 89], [0, 1, 45], [1, 0, 3], [1, 0, 4]])
    orow, lrow = oracle.attention_rows(q, k, v, 0.5, idx, workers=2)
    for r, (b, h, i) in enumerate(idx):
        np.testing.assert_allclose(orow[r], o[b, h, i], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lrow[r], lse[b, h, i], rtol=1e-15, atol=1e-15)


def test_empty_sequence():
    q = np.zeros((1, 2, 0, 8))
    o, lse = oracle.attention(q, q, q, 1.0)
    assert o.shape == (1, 2, 0, 8) and lse.shape == (1, 2, 0)


def test_nan_key_poisons_its_head_only():
    q, k, v = _rand(1, 2, 6, 4, 23)
    k[0, 0, 3, 1] = np.nan
    with np.errstate(invalid="ignore"):
        o, lse = _attn(q, k, v, 1.0)
    assert np.all(np.isnan(o[0, 0])) and np.all(np.isnan(lse[0, 0]))
    assert np.all(np.isfinite(o[0, 1])) and np.all(np.isfinite(lse[0, 1]))


# --------------------------------------------------------------------------
# planted mistakes: every one must fail at least one pin
# --------------------------------------------------------------------------

def _mut_no_scale(q, k, v, scale):
    s = q @ k.T
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def _mut_scale_squared(q, k, v, scale):
    s = scale * scale * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def _mut_transposed_scores(q, k, v, scale):
    s = scale * (q @ k.T)
    if s.shape[0] == s.shape[1]:
        s = s.T
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def _mut_max_wrong_axis(q, k, v, scale):
    s = scale * (q @ k.T)
    m = s.max(0, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    mm = s.max(1)
    return (p @ v) / l, mm + np.log(l[:, 0])


def _mut_sum_wrong_axis(q, k, v, scale):
    s = scale * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(s - m)
    l = p.sum(0)[: p.shape[0], None] if p.shape[0] <= p.shape[1] else p.sum(1, keepdims=True) * 2
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def _mut_exp_sign(q, k, v, scale):
    s = scale * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(m - s); l = p.sum(1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def _mut_no_max_subtraction(q, k, v, scale):
    s = scale * (q @ k.T)
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(s); l = p.sum(1, keepdims=True)
        return (p @ v) / l, np.log(l[:, 0])


def _mut_unnormalised(q, k, v, scale):
    s = scale * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return p @ v, m[:, 0] + np.log(l[:, 0])


def _mut_lse_without_max(q, k, v, scale):
    s = scale * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return (p @ v) / l, np.log(l[:, 0])


def _mut_lse_log2(q, k, v, scale):
    s = scale * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log2(l[:, 0])


def _mut_drop_last_key(q, k, v, scale):
    k, v = k[:-1], v[:-1]
    s = scale * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def _mut_v_shifted(q, k, v, scale):
    v = np.roll(v, 1, axis=0)
    s = scale * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def _mut_keys_cut_to_queries(q, k, v, scale):
    # confuses the key count with the query count (invisible when they are equal)
    k, v = k[:q.shape[0]], v[:q.shape[0]]
    s = scale * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def _mut_sqrt_scale(q, k, v, scale):
    s = math.sqrt(abs(scale)) * (q @ k.T)
    m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


MUTANTS = [_mut_no_scale, _mut_scale_squared, _mut_transposed_scores, _mut_max_wrong_axis,
           _mut_sum_wrong_axis, _mut_exp_sign, _mut_no_max_subtraction, _mut_unnormalised,
           _mut_lse_without_max, _mut_lse_log2, _mut_drop_last_key, _mut_v_shifted,
           _mut_sqrt_scale, _mut_keys_cut_to_queries]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    """Plant a mistake in the oracle (on the CPU) and check some pin fails."""
    monkeypatch.setattr(attention_mod, "_rows", mutant)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(_attn)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutant.__name__}"


def _online_no_alpha_on_acc(q, k, v, scale, block_n):
    B, H, N, _ = q.shape
    o = np.empty(v.shape); lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf); l = np.zeros(N); acc = np.zeros((N, v.shape[-1]))
            for j0 in range(0, N, block_n):
                s = scale * (q[b, h] @ k[b, h, j0:j0 + block_n].T)
                m_new = np.maximum(m, s.max(1)); p = np.exp(s - m_new[:, None])
                alpha = np.exp(m - m_new)
                l = alpha * l + p.sum(1)
                acc = acc + p @ v[b, h, j0:j0 + block_n]  # mistake: acc not rescaled
                m = m_new
            o[b, h] = acc / l[:, None]; lse[b, h] = m + np.log(l)
    return o, lse


def test_online_mistake_is_caught():
    q, k, v = _rand(1, 1, 130, 8, 5)
    k[..., ::9, :] *= 8.0
    o, lse = _attn(q, k, v, 0.6)
    o2, _ = _online_no_alpha_on_acc(q, k, v, 0.6, 64)
    assert not np.allclose(o, o2, rtol=1e-6, atol=1e-6)


# --------------------------------------------------------------------------
# causal variant: query i attends keys 0..i (page 1 section 4's causal mask,
# page 3 section 3's masked_fill before the softmax, page 3 section 5's
# ``causal`` flag)
# --------------------------------------------------------------------------

def _attn_causal(q, k, v, scale):
    return oracle.attention(q, k, v, scale, causal=True, workers=1)


def cpin_brute_force(attn):
    """Pure-Python textbook softmax over the keys j <= i only."""
    for (N, d, seed) in [(1, 1, 30), (2, 4, 31), (5, 4, 32), (17, 8, 33), (17, 1, 34)]:
        q, k, v = _rand(1, 2, N, d, seed)
        o, lse = attn(q, k, v, 0.8)
        for h in range(2):
            Q, K, V = q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist()
            for i in range(N):
                ob, lb = _brute_row(Q[i], K[:i + 1], V[:i + 1], 0.8)
                np.testing.assert_allclose(o[0, h, i], ob, rtol=1e-12, atol=1e-12)
                assert abs(lse[0, h, i] - lb) <= 1e-12 * max(1.0, abs(lb))


def cpin_prefix(attn):
    """Row i equals the unmasked definition on the prefix K[:i+1], V[:i+1]."""
    q, k, v = _rand(2, 2, 40, 8, 35)
    o, lse = attn(q, k, v, 0.5)
    for i in (0, 1, 7, 20, 39):
        op, lp = _attn(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.5)
        np.testing.assert_allclose(o[:, :, i], op[:, :, i], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], lp[:, :, i], rtol=1e-13, atol=1e-13)


def cpin_first_row(attn):
    """Closed form: row 0 sees only key 0, so O = v_0 and lse = scale * q_0 . k_0."""
    q, k, v = _rand(1, 3, 12, 6, 36)
    o, lse = attn(q, k, v, 0.3)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=1e-14, atol=1e-14)


def cpin_sdpa(attn):
    for (B, H, N, d, seed, scale) in [(2, 3, 33, 16, 37, 0.25), (1, 2, 70, 64, 38, 0.125)]:
        q, k, v = _rand(B, H, N, d, seed)
        o, lse = attn(q, k, v, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale,
                                                               is_causal=True)
        s = scale * (tq @ tk.transpose(-1, -2))
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        np.testing.assert_allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def cpin_weights(attn):
    """With V = I the outputs are the weights: rows sum to one, zero above the diagonal."""
    N = 23
    q, k, _ = _rand(1, 1, N, 6, 39)
    o, _ = attn(q, k, np.eye(N)[None, None], 0.9)
    np.testing.assert_allclose(o.sum(axis=-1), 1.0, atol=1e-12)
    assert np.all(o[0, 0][np.triu(np.ones((N, N), dtype=bool), 1)] == 0.0)
    assert np.all(np.diag(o[0, 0]) > 0.0)
    np.testing.assert_allclose(o[0, 0], oracle.softmax_probs(q[0, 0], k[0, 0], 0.9, causal=True),
                               atol=1e-13)


def cpin_online_matches(attn):
    for (N, bn) in [(50, 1), (50, 7), (130, 64), (33, 33)]:
        q, k, v = _rand(1, 2, N, 8, 140 + N + bn)
        k[..., ::9, :] *= 8.0
        o, lse = attn(q, k, v, 0.6)
        o2, lse2 = attention_online(q, k, v, 0.6, bn, causal=True)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-12)


CAUSAL_PINS = [cpin_brute_force, cpin_prefix, cpin_first_row, cpin_sdpa, cpin_weights,
               cpin_online_matches]


@pytest.mark.parametrize("pin", CAUSAL_PINS, ids=lambda p: p.__name__)
def test_causal_oracle_pin(pin):
    pin(_attn_causal)


def test_causal_attention_rows_matches_full():
    q, k, v = _rand(2, 2, 90, 8, 40)
    o, lse = oracle.attention(q, k, v, 0.5, causal=True, workers=1, row_chunk=32)
    idx = np.array([[0, 0, 0], [1, 1, 89], [0, 1, 45], [1, 0, 3], [1, 0, 33]])
    orow, lrow = oracle.attention_rows(q, k, v, 0.5, idx, causal=True, workers=2)
    for r, (b, h, i) in enumerate(idx):
        np.testing.assert_allclose(orow[r], o[b, h, i], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lrow[r], lse[b, h, i], rtol=1e-15, atol=1e-15)


def _cmut(mask_fn):
    """A copy of the row kernel whose causal mask is ``mask_fn(j, i) -> masked``."""
    def rows_fn(q, k, v, scale, rows=None):
        s = scale * (q @ k.T)
        if rows is not None:
            s[mask_fn(np.arange(k.shape[0])[None, :], np.asarray(rows)[:, None])] = -np.inf
        m = s.max(1, keepdims=True); p = np.exp(s - m); l = p.sum(1, keepdims=True)
        return (p @ v) / l, m[:, 0] + np.log(l[:, 0])
    return rows_fn


CAUSAL_MUTANTS = {
    "no_mask": _cmut(lambda j, i: np.zeros(np.broadcast(j, i).shape, dtype=bool)),
    "diagonal_masked": _cmut(lambda j, i: j >= i),
    "transposed_mask": _cmut(lambda j, i: j < i),
    "row_index_off_by_one": _cmut(lambda j, i: j > i + 1),
    "row_index_shifted_down": _cmut(lambda j, i: j > i - 1 + (i == 0)),
}


@pytest.mark.parametrize("name", sorted(CAUSAL_MUTANTS))
def test_causal_planted_mistakes_are_caught(name, monkeypatch):
    monkeypatch.setattr(attention_mod, "_rows", CAUSAL_MUTANTS[name])
    caught = []
    for pin in CAUSAL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(_attn_causal)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no causal pin caught {name}"


def test_cross_length_shape_rules():
    """N queries against Nk keys: o and lse follow q; no keys, a causal mask
    over unequal lengths and mismatched k/v rows are refused."""
    q, k, v = _rand_kv(1, 2, 3, 11, 4, 40)
    o, lse = oracle.attention(q, k, v, 0.5)
    assert o.shape == (1, 2, 3, 4) and lse.shape == (1, 2, 3)
    with pytest.raises(ValueError):
        oracle.attention(q, k[:, :, :0], v[:, :, :0], 0.5)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 0.5, causal=True)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v[:, :, :5], 0.5)
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, v, 0.5, [[0, 0, 0]], causal=True)
    with pytest.raises(ValueError):
        attention_online(q, k, v, 0.5, 4, causal=True)
    idx = np.array([[0, 1, 2], [0, 0, 0]])
    orow, lrow = oracle.attention_rows(q, k, v, 0.5, idx)
    np.testing.assert_allclose(orow, o[0, [1, 0], [2, 0]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lrow, lse[0, [1, 0], [2, 0]], rtol=1e-15, atol=1e-15)
