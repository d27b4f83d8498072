"""The entry points under HIP graph capture.

Every entry point only enqueues kernels on the caller's stream (no allocation,
no synchronisation, no memset), so torch can capture it into a graph.  Each
test captures a call, then replays the graph several times with new input
values written into the captured buffers between replays (eager work and a
synchronisation in between), and checks every replay bit for bit against an
eager call on the same inputs: the kernels are deterministic, so a replay that
read stale inputs or skipped a node would differ.
"""
import pytest

import datagen

torch = pytest.importorskip("torch")
aa = pytest.importorskip("attention_attn_fwd_07_amd")

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _inputs(seed, B, H, N, d, dtype):
    q, k, v = datagen.make_qkv(B, H, N, d, dtype, seed)
    return [t.to("cuda") for t in (q, k, v)]


def _refill(bufs, seed, dtype):
    """Write fresh values into the captured buffers in place (eager work)."""
    B, H, N, d = bufs[0].shape
    fresh = _inputs(seed, B, H, N, d, dtype) + _inputs(seed + 7, B, H, N, d, dtype)
    for b, f in zip(bufs, fresh):
        b.copy_(f)


@pytest.mark.parametrize("d,causal", [(64, False), (128, False), (128, True)])
def test_forward_graph_replays(d, causal):
    B, H, N = 2, 3, 300
    q, k, v = _inputs(11, B, H, N, d, "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = d ** -0.5
    aa.attn_fwd(q, k, v, o, lse, scale, causal=causal)  # loads the library
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        aa.attn_fwd(q, k, v, o, lse, scale, causal=causal)
    for r in range(REPLAYS):
        _refill((q, k, v), 100 + r, "bf16")
        g.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        o.zero_()
        lse.zero_()
        aa.attn_fwd(q, k, v, o, lse, scale, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o), f"replay {r}: O differs from the eager call"
        assert torch.equal(lse_g, lse), f"replay {r}: lse differs from the eager call"


def test_splitkv_graph_replays():
    B, H, N, d, S = 1, 4, 700, 128, 3
    q, k, v = _inputs(12, B, H, N, d, "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(aa.splitkv_workspace_size(B, H, N, d, S) // 4, dtype=torch.float32,
                     device="cuda")
    scale = d ** -0.5
    aa.plan(q, k, v, o, lse, scale, splits=S, workspace=ws)()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        aa.plan(q, k, v, o, lse, scale, splits=S, workspace=ws)()
    for r in range(REPLAYS):
        _refill((q, k, v), 200 + r, "bf16")
        g.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        o.zero_()
        lse.zero_()
        ws.zero_()
        aa.plan(q, k, v, o, lse, scale, splits=S, workspace=ws)()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o), f"replay {r}: O differs from the eager call"
        assert torch.equal(lse_g, lse), f"replay {r}: lse differs from the eager call"


def test_decode_splitkv_graph_replays():
    """One query per head against 3000 keys (the decode kernel) through the
    split-KV path, captured and replayed."""
    B, H, N, Nk, d, S = 2, 4, 1, 3000, 128, 8
    q, k, v = (t.to("cuda") for t in datagen.make_qkv_kv(B, H, N, Nk, d, "bf16", 13))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(aa.splitkv_workspace_size(B, H, N, d, S, Nk) // 4, dtype=torch.float32,
                     device="cuda")
    scale = d ** -0.5
    aa.plan(q, k, v, o, lse, scale, splits=S, workspace=ws)()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        aa.plan(q, k, v, o, lse, scale, splits=S, workspace=ws)()
    for r in range(REPLAYS):
        fresh = datagen.make_qkv_kv(B, H, N, Nk, d, "bf16", 300 + r)
        for b, f in zip((q, k, v), fresh):
            b.copy_(f.to("cuda"))
        g.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        o.zero_()
        lse.zero_()
        ws.zero_()
        aa.plan(q, k, v, o, lse, scale, splits=S, workspace=ws)()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o), f"replay {r}: O differs from the eager call"
        assert torch.equal(lse_g, lse), f"replay {r}: lse differs from the eager call"


@pytest.mark.parametrize("dtype,causal", [("bf16", False), ("bf16", True), ("f32", True)])
def test_backward_graph_replays(dtype, causal):
    B, H, N, d = 1, 2, 260, 64
    q, k, v = _inputs(13, B, H, N, d, dtype)
    do = datagen.make_grad(B, H, N, d, dtype, 14).to("cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(aa.bwd_workspace_size(B, H, N, d) // 4, dtype=torch.float32,
                     device="cuda")
    scale = d ** -0.5

    def step():
        aa.attn_fwd(q, k, v, o, lse, scale, causal=causal)
        aa.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, scale, ws, causal=causal)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        _refill((q, k, v, do), 300 + r, dtype)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        for t in (o, lse, dq, dk, dv, ws):
            t.zero_()
        step()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "lse", "dQ", "dK", "dV"), got, (o, lse, dq, dk, dv)):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"


def test_merge_graph_replays():
    """Forwards over three key shards and their merge (attn_fwd_merge),
    captured together and replayed."""
    B, H, N, Nk, d = 1, 3, 40, 900, 128
    q, k, v = (t.to("cuda") for t in datagen.make_qkv_kv(B, H, N, Nk, d, "bf16", 15))
    shards = [(0, 250), (250, 700), (700, 900)]
    ks = [k[:, :, a:b].contiguous() for a, b in shards]
    vs = [v[:, :, a:b].contiguous() for a, b in shards]
    parts = [(torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda"))
             for _ in shards]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = d ** -0.5

    def step():
        for kk, vv, (po, pl) in zip(ks, vs, parts):
            aa.attn_fwd(q, kk, vv, po, pl, scale)
        aa.merge([p[0] for p in parts], [p[1] for p in parts], o, lse)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        fq, fk, fv = datagen.make_qkv_kv(B, H, N, Nk, d, "bf16", 400 + r)
        q.copy_(fq.to("cuda"))
        for (a, b), kk, vv in zip(shards, ks, vs):
            kk.copy_(fk[:, :, a:b].to("cuda"))
            vv.copy_(fv[:, :, a:b].to("cuda"))
        g.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        o.zero_()
        lse.zero_()
        step()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o), f"replay {r}: O differs from the eager call"
        assert torch.equal(lse_g, lse), f"replay {r}: lse differs from the eager call"
