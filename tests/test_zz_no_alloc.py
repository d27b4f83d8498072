"""The allocation-free split-KV entry point, attn_fwd_splitkv_static, through
the C ABI: its output against attn_fwd_splitkv's (caller workspace) on the
same inputs and splits, on two calls in a row, the second with a smaller
input (the library's static array keeps the first call's contents), and both
against the fp64 oracle at the stated bars.  Runs alone in a fresh process
as well as after the other tests."""
import ctypes
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from test_parity import check

pytestmark = pytest.mark.gpu

STATIC_LIMIT = -13


def _lib():
    import attention_attn_fwd_07_amd as attn
    lib = ctypes.CDLL(attn.library_path())
    lib.attn_fwd_splitkv_static.argtypes = [ctypes.POINTER(attn._Args), ctypes.c_int]
    lib.attn_fwd_splitkv_static.restype = ctypes.c_int
    lib.attn_fwd_splitkv.argtypes = [ctypes.POINTER(attn._Args), ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_size_t]
    lib.attn_fwd_splitkv.restype = ctypes.c_int
    lib.attn_fwd_splitkv_workspace.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.attn_fwd_splitkv_workspace.restype = ctypes.c_size_t
    return attn, lib


def _args(attn, q, k, v, o, lse, scale, dtype_code, stream):
    a = attn._Args()
    a.q, a.k, a.v, a.o, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr()
    a.B, a.H, a.N, a.d = (int(x) for x in q.shape)
    a.scale, a.dtype, a.flags = scale, dtype_code, 0
    a.q_stride[:] = a.k_stride[:] = a.v_stride[:] = a.o_stride[:] = (0, 0, 0)
    a.stream = stream
    return a


CASES = [  # (B, H, N, d, dtype, splits): the second is smaller than the first
    (2, 4, 1000, 128, "bf16", 3),
    (1, 2, 300, 64, "f16", 2),
]


def test_static_matches_workspace_call_twice_in_a_row():
    attn, lib = _lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    code = {"f32": 0, "f16": 1, "bf16": 2}
    for B, H, N, d, dtype, splits in CASES:
        what = f"B{B} H{H} N{N} d{d} {dtype} S={splits}"
        print(what, flush=True)
        q, k, v = datagen.make_qkv(B, H, N, d, dtype, seed=900 + N)
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        scale = 1.0 / math.sqrt(d)
        o_s = torch.full_like(qd, float("nan"))
        l_s = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
        a = _args(attn, qd, kd, vd, o_s, l_s, scale, code[dtype], stream)
        assert lib.attn_fwd_splitkv_static(ctypes.byref(a), splits) == 0
        o_w = torch.full_like(qd, float("nan"))
        l_w = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
        nbytes = lib.attn_fwd_splitkv_workspace(B, H, N, d, splits)
        assert 0 < nbytes <= attn.STATIC_WORKSPACE_BYTES
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
        b = _args(attn, qd, kd, vd, o_w, l_w, scale, code[dtype], stream)
        assert lib.attn_fwd_splitkv(ctypes.byref(b), splits, ws.data_ptr(), nbytes) == 0
        torch.cuda.synchronize()
        # the same kernels on the same inputs: bit-identical results
        assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16)), what
        assert torch.equal(l_s, l_w), what
        o_ref, lse_ref = oracle.attention(q, k, v, scale)
        check(o_s.cpu().double().numpy(), l_s.cpu().double().numpy(), o_ref, lse_ref, dtype, what)


def test_static_rejects_sizes_beyond_the_array():
    attn, lib = _lib()
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 64, 1024, 128, dtype=torch.bfloat16, device=dev)
    k, v, o = q.clone(), q.clone(), q.clone()
    lse = torch.zeros(1, 64, 1024, dtype=torch.float32, device=dev)
    # 64 heads x 1024 rows x 129 floats x 3 splits = 101 MB > 64 MiB
    assert lib.attn_fwd_splitkv_workspace(1, 64, 1024, 128, 3) > attn.STATIC_WORKSPACE_BYTES
    a = _args(attn, q, k, v, o, lse, 0.1, 2, torch.cuda.current_stream(dev).cuda_stream)
    assert lib.attn_fwd_splitkv_static(ctypes.byref(a), 3) == STATIC_LIMIT
    with pytest.raises(ValueError):
        attn.attn_fwd_splitkv_static(q, k, v, o, lse, 0.1, 3)
    # one split fits (33.8 MB): the binding's call succeeds and matches attn_fwd
    attn.attn_fwd_splitkv_static(q, k, v, o, lse, 0.1, 1)
    o2, l2 = attn.fwd(q, k, v, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
