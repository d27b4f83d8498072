"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments before making any HIP call."""
import ctypes
import glob
import os
import re

import pytest

from attention_attn_fwd_07_amd import build as build_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULLPTR, SHAPE, HEAD_DIM, DTYPE, SCALE, ALIGN, ALIAS, HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8
F32, F16, BF16 = 0, 1, 2


@pytest.fixture(scope="module")
def lib():
    path = build_mod.ensure_built()
    l = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    l.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                           ctypes.c_int, vp]
    l.attn_fwd.restype = ctypes.c_int
    l.attn_strerror.argtypes = [ctypes.c_int]
    l.attn_strerror.restype = ctypes.c_char_p
    return l


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \t\*]*?\b([A-Za-z_]\w*)\s*\([^;{]*\)\s*;", text,
                            flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    assert {"attn_fwd", "attn_strerror", "attn_version"} <= set(declared_functions())


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_version_and_strerror(lib):
    lib.attn_version.restype = ctypes.c_int
    assert lib.attn_version() >= 100
    for code in (OK, NULLPTR, SHAPE, HEAD_DIM, DTYPE, SCALE, ALIGN, ALIAS, HIP, 12345):
        assert lib.attn_strerror(code)


# distinct, 16-byte aligned fake device addresses; validation never touches them
Q, K, V, O, L = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def call(lib, q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=128, d=64, scale=0.125, dtype=BF16):
    return lib.attn_fwd(q, k, v, o, lse, B, H, N, d, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), SHAPE), (dict(H=-3), SHAPE), (dict(N=-1), SHAPE), (dict(d=-64), SHAPE),
    (dict(dtype=3), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(d=32), HEAD_DIM), (dict(d=96), HEAD_DIM), (dict(d=256), HEAD_DIM), (dict(d=0), HEAD_DIM),
    (dict(scale=float("nan")), SCALE), (dict(scale=float("inf")), SCALE),
    (dict(scale=float("-inf")), SCALE),
    (dict(q=None), NULLPTR), (dict(k=None), NULLPTR), (dict(v=None), NULLPTR),
    (dict(o=None), NULLPTR),
    (dict(q=Q + 8), ALIGN), (dict(o=O + 2), ALIGN), (dict(v=V + 4), ALIGN), (dict(lse=L + 2), ALIGN),
    (dict(o=Q), ALIAS), (dict(o=K + 64), ALIAS), (dict(lse=V), ALIAS), (dict(lse=O + 16), ALIAS),
    (dict(N=(1 << 22) + 1), SHAPE),
    (dict(B=1 << 40, H=1 << 30), SHAPE),
])
def test_rejects_before_any_hip_call(lib, kw, code):
    assert call(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(N=0, q=None, o=None),
                                dict(B=0, d=128, dtype=F32)])
def test_empty_is_a_no_op(lib, kw):
    assert call(lib, **kw) == OK


def test_shape_checked_before_emptiness(lib):
    # bad head dim or dtype is an error even for empty input
    assert call(lib, N=0, d=80) == HEAD_DIM
    assert call(lib, N=0, dtype=7) == DTYPE


def test_python_binding_rejects_cpu_tensors():
    import torch
    import attention_attn_fwd_07_amd as attn
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.attn_fwd(q, q, q, torch.empty_like(q), None, 0.125)


# ---------------------------------------------------------------------------
# attn_fwd_ex: flags and strides
# ---------------------------------------------------------------------------

FLAGS, LAYOUT = -9, -10


def ex_args(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=128, d=64, scale=0.125, dtype=BF16,
            flags=0, qs=(0, 0, 0), ks=(0, 0, 0), vs=(0, 0, 0), os_=(0, 0, 0), Nk=0):
    from attention_attn_fwd_07_amd import _Args
    a = _Args()
    a.q, a.k, a.v, a.o, a.lse = q, k, v, o, lse
    a.B, a.H, a.N, a.d, a.scale, a.dtype, a.flags = B, H, N, d, scale, dtype, flags
    a.Nk = Nk
    a.q_stride[:], a.k_stride[:], a.v_stride[:], a.o_stride[:] = qs, ks, vs, os_
    a.stream = None
    return a


def call_ex(lib, **kw):
    from attention_attn_fwd_07_amd import _Args
    lib.attn_fwd_ex.argtypes = [ctypes.POINTER(_Args)]
    lib.attn_fwd_ex.restype = ctypes.c_int
    return lib.attn_fwd_ex(ctypes.byref(ex_args(**kw)))


def test_args_struct_matches_the_header(tmp_path):
    """The binding's ctypes mirror of attn_fwd_args_t has the C layout."""
    import shutil
    import subprocess
    from attention_attn_fwd_07_amd import _Args
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in _Args._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "attn_fwd.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(attn_fwd_args_t));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(attn_fwd_args_t, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(_Args)
    assert got[1:] == [getattr(_Args, f).offset for f in fields]


def test_ex_null_args(lib):
    lib.attn_fwd_ex.argtypes = [ctypes.c_void_p]
    lib.attn_fwd_ex.restype = ctypes.c_int
    assert lib.attn_fwd_ex(None) == NULLPTR


@pytest.mark.parametrize("kw,code", [
    (dict(flags=2), FLAGS), (dict(flags=0x80000001), FLAGS),
    (dict(qs=(0, 0, -64)), LAYOUT), (dict(ks=(2 * 128 * 64, 128 * 64, 60)), LAYOUT),
    (dict(vs=(-8, 8, 64)), LAYOUT), (dict(os_=(2 * 128 * 64, 128 * 64, 32)), LAYOUT),
    # o rows of different heads collide: head stride 32 < d = 64
    (dict(os_=(2 * 128 * 128, 32, 128)), LAYOUT),
    # o rows of the two batches collide: batch stride 32 < d = 64
    (dict(B=2, os_=(32, 128 * 256, 256)), LAYOUT),
    (dict(B=0, flags=2), FLAGS),
    (dict(N=0, qs=(0, 0, 3)), OK),   # empty input returns before strides are looked at
    (dict(q=None, flags=1), NULLPTR),
])
def test_ex_rejects_before_any_hip_call(lib, kw, code):
    assert call_ex(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(Nk=-1), SHAPE), (dict(Nk=(1 << 22) + 1), SHAPE),
    # the causal mask is defined for one sequence length only
    (dict(Nk=4096, flags=1), FLAGS), (dict(N=1, Nk=128, flags=1), FLAGS),
    # k spans its own Nk rows: 2 heads x 4096 keys x 64 x 2 bytes = 1 MiB from K,
    # so an o placed half-way through it aliases k (it would not with Nk = N)
    (dict(Nk=4096, o=K + (1 << 19)), ALIAS), (dict(Nk=4096, lse=K + (1 << 19)), ALIAS),
    # k's explicit strides are checked over Nk rows: a head of 2^20 keys with a
    # row stride of 2048 elements is beyond 32-bit byte offsets
    (dict(N=16, Nk=1 << 20, ks=(0, 0, 2048), **{"k": 1 << 40}), SHAPE),
    (dict(N=0, Nk=4096), OK), (dict(B=0, Nk=-5), SHAPE),
])
def test_ex_key_length_rejects_before_any_hip_call(lib, kw, code):
    assert call_ex(lib, **kw) == code


def test_rows_disjoint_interleaved_heads_are_valid():
    # [B, N, H, d] viewed as [B, H, N, d]: head stride d, row stride H d.  A
    # valid layout, accepted by the host checks (it would launch, so only the
    # disjointness logic is exercised here, through the Python stride helper).
    import torch
    from attention_attn_fwd_07_amd import _strides
    t = torch.zeros(1, 128, 2, 64).transpose(1, 2)
    assert _strides(t) == (128 * 2 * 64, 64, 128)


def test_broadcast_row_has_no_stride_triple():
    # a single row expanded to [B, H, N, d] has leading strides (0, 0, 0), the
    # ABI's contiguous mark: inputs are copied, outputs rejected, and the
    # stride helper never passes (0, 0, 0) for a non-contiguous tensor
    import torch
    from attention_attn_fwd_07_amd import _strides, _unbroadcast
    row = torch.arange(64, dtype=torch.float32).reshape(1, 1, 1, 64)
    t = row.expand(2, 3, 5, 64)
    assert not t.is_contiguous() and tuple(t.stride()[:3]) == (0, 0, 0)
    c = _unbroadcast(t, "k")
    assert c.is_contiguous() and torch.equal(c, t) and _strides(c) == (0, 0, 0)
    with pytest.raises(ValueError):
        _unbroadcast(t, "o", output=True)
    with pytest.raises(ValueError):
        _strides(t)
    # other views pass through unchanged
    u = torch.zeros(1, 5, 2, 64).transpose(1, 2)
    assert _unbroadcast(u, "q") is u


def test_ex_strided_alias_uses_the_strided_extent(lib):
    # o written with BNHD strides spans 2*128*64 elements; an lse placed inside
    # that span is an alias even though it lies beyond o's first head.
    bnhd = (128 * 2 * 64, 64, 2 * 64)
    assert call_ex(lib, os_=bnhd, lse=O + 2 * 64 * 2 * 100) == ALIAS


def test_ex_head_bytes_limit(lib):
    # a head's rows must be addressable with 32-bit byte offsets in the kernels
    assert call_ex(lib, N=1 << 20, ks=(0, 0, 2048), d=64) == SHAPE


@pytest.mark.parametrize("stride", [(1 << 63) // 6 // 8 * 8, (1 << 62) // 8 * 8 - 8,
                                    (1 << 61) // 8 * 8])
def test_ex_huge_row_stride_is_rejected(lib, stride):
    # fp32, N = 2 and a row stride near INT64_MAX / 6: N * stride * 4 overflows
    # int64; the head-bytes check must still reject it (no wrap past the bound)
    code = call_ex(lib, B=1, H=1, N=2, d=64, dtype=F32, ks=(0, 0, stride))
    assert code in (SHAPE, LAYOUT)


# ---------------------------------------------------------------------------
# attn_fwd_splitkv: argument checks and workspace sizing
# ---------------------------------------------------------------------------

SPLITS, WORKSPACE = -11, -12
W = 0x40000000  # fake, 16-byte aligned workspace address far from the tensors


def call_split(lib, splits=4, ws=W, ws_bytes=1 << 30, **kw):
    from attention_attn_fwd_07_amd import _Args
    lib.attn_fwd_splitkv.argtypes = [ctypes.POINTER(_Args), ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_size_t]
    lib.attn_fwd_splitkv.restype = ctypes.c_int
    return lib.attn_fwd_splitkv(ctypes.byref(ex_args(**kw)), splits, ws, ws_bytes)


def ws_size(lib, B, H, N, d, splits):
    lib.attn_fwd_splitkv_workspace.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.attn_fwd_splitkv_workspace.restype = ctypes.c_size_t
    return lib.attn_fwd_splitkv_workspace(B, H, N, d, splits)


@pytest.mark.parametrize("B,H,N,d,splits,used", [
    (1, 8, 65536, 64, 4, 4), (2, 3, 1000, 128, 7, 6),   # 16 tiles: 3 per split -> 6 splits
    (1, 1, 100, 64, 8, 2), (1, 1, 64, 128, 5, 1), (4, 2, 129, 64, 64, 3)])
def test_workspace_size_counts_non_empty_splits(lib, B, H, N, d, splits, used):
    assert ws_size(lib, B, H, N, d, splits) == used * B * H * N * (d + 1) * 4


@pytest.mark.parametrize("args", [(1, 1, 0, 64, 2), (1, 1, 10, 64, 0), (1, 1, 10, 64, 65),
                                  (1, 1, 10, 96, 2), (-1, 1, 10, 64, 2)])
def test_workspace_size_zero_for_invalid(lib, args):
    assert ws_size(lib, *args) == 0


def ws_size_ex(lib, B, H, N, Nk, d, splits):
    lib.attn_fwd_splitkv_workspace_ex.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int]
    lib.attn_fwd_splitkv_workspace_ex.restype = ctypes.c_size_t
    return lib.attn_fwd_splitkv_workspace_ex(B, H, N, Nk, d, splits)


@pytest.mark.parametrize("B,H,N,Nk,d,splits,used", [
    (1, 32, 1, 65536, 128, 16, 16), (2, 8, 4, 1000, 64, 7, 6),   # 16 key tiles -> 6 splits
    (1, 2, 3000, 100, 64, 8, 2), (1, 1, 1, 1, 128, 5, 1)])
def test_workspace_size_ex_counts_splits_of_the_keys(lib, B, H, N, Nk, d, splits, used):
    # partial results are per query row; the number of splits follows the keys
    assert ws_size_ex(lib, B, H, N, Nk, d, splits) == used * B * H * N * (d + 1) * 4


def test_workspace_size_ex_zero_key_length_means_n(lib):
    for (B, H, N, d, splits) in [(1, 8, 65536, 64, 4), (2, 3, 1000, 128, 7), (1, 1, 0, 64, 2)]:
        assert ws_size_ex(lib, B, H, N, 0, d, splits) == ws_size(lib, B, H, N, d, splits)
        assert ws_size_ex(lib, B, H, N, N, d, splits) == ws_size(lib, B, H, N, d, splits)
    assert ws_size_ex(lib, 1, 1, 10, -1, 64, 2) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(splits=0), SPLITS), (dict(splits=65), SPLITS), (dict(splits=-2), SPLITS),
    (dict(flags=1), FLAGS),
    (dict(ws=None), NULLPTR), (dict(ws=W + 4), ALIGN),
    (dict(ws_bytes=4 * 2 * 128 * 65 * 2 - 4), WORKSPACE),  # 2 tiles -> 2 splits used
    (dict(ws=O), ALIAS), (dict(ws=L - 1024 * 16), ALIAS), (dict(ws=Q + 64), ALIAS),
    (dict(N=0), OK), (dict(N=0, ws=None), OK),
    # one query row against 4096 keys: 64 key tiles, 4 splits of one row each
    (dict(N=1, Nk=4096, ws_bytes=4 * 2 * 1 * 65 * 4 - 4, k=1 << 40, v=2 << 40), WORKSPACE),
    (dict(N=1, Nk=4096, flags=1, k=1 << 40, v=2 << 40), FLAGS),
])
def test_splitkv_rejects_before_any_hip_call(lib, kw, code):
    assert call_split(lib, **kw) == code


STATIC_LIMIT = -13
# fake tensors far apart, for shapes whose extents exceed the 1 MiB spacing above
FAR = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40, lse=5 << 40)


def call_static(lib, splits=4, **kw):
    from attention_attn_fwd_07_amd import _Args
    lib.attn_fwd_splitkv_static.argtypes = [ctypes.POINTER(_Args), ctypes.c_int]
    lib.attn_fwd_splitkv_static.restype = ctypes.c_int
    return lib.attn_fwd_splitkv_static(ctypes.byref(ex_args(**kw)), splits)


@pytest.mark.parametrize("kw,code", [
    # the partial results of 8 splits of 64 x 65536 rows are far beyond 64 MiB
    (dict(B=1, H=64, N=65536, d=128, splits=8, **FAR), STATIC_LIMIT),
    (dict(B=1, H=64, N=1024, d=128, splits=3, **FAR), STATIC_LIMIT),   # 101 MB
    (dict(splits=0), SPLITS), (dict(splits=65), SPLITS), (dict(flags=1), FLAGS),
    (dict(d=96), HEAD_DIM), (dict(q=None), NULLPTR), (dict(o=Q), ALIAS),
    (dict(N=0), OK),
])
def test_splitkv_static_rejects_before_any_hip_call(lib, kw, code):
    assert call_static(lib, **kw) == code


def test_splitkv_static_null_args(lib):
    lib.attn_fwd_splitkv_static.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.attn_fwd_splitkv_static.restype = ctypes.c_int
    assert lib.attn_fwd_splitkv_static(None, 2) == NULLPTR


# ---------------------------------------------------------------------------
# attn_fwd_merge: argument checks
# ---------------------------------------------------------------------------

def call_merge(lib, nparts=2, o_parts=None, lse_parts=None, o=O, lse=L, B=1, H=2, N=128, d=64,
               dtype=BF16, null_arrays=False):
    vp = ctypes.c_void_p
    lib.attn_fwd_merge.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int, vp, vp,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, vp]
    lib.attn_fwd_merge.restype = ctypes.c_int
    if o_parts is None:
        o_parts = [(1 + s) << 36 for s in range(max(nparts, 0))]
    if lse_parts is None:
        lse_parts = [(100 + s) << 36 for s in range(max(nparts, 0))]
    n = max(len(o_parts), 1)
    op = (vp * n)(*o_parts) if not null_arrays else None
    lp = (vp * n)(*lse_parts) if not null_arrays else None
    return lib.attn_fwd_merge(op, lp, nparts, o, lse, B, H, N, d, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(nparts=0), SPLITS), (dict(nparts=65), SPLITS), (dict(nparts=-1), SPLITS),
    (dict(dtype=9), DTYPE), (dict(d=96), HEAD_DIM), (dict(N=-2), SHAPE),
    (dict(null_arrays=True), NULLPTR), (dict(o=None), NULLPTR),
    (dict(o_parts=[1 << 36, None]), NULLPTR), (dict(lse_parts=[100 << 36, None]), NULLPTR),
    (dict(o=O + 8), ALIGN), (dict(lse=L + 2), ALIGN), (dict(o_parts=[(1 << 36) + 8, 2 << 36]), ALIGN),
    (dict(lse_parts=[(100 << 36) + 2, 101 << 36]), ALIGN),
    (dict(o=(1 << 36) + 64), ALIAS), (dict(lse=(101 << 36) + 4), ALIAS),
    (dict(lse=O + 16), ALIAS), (dict(o=(100 << 36) + 16), ALIAS),
    (dict(N=0), OK), (dict(B=0, null_arrays=True), OK),
])
def test_merge_rejects_before_any_hip_call(lib, kw, code):
    assert call_merge(lib, **kw) == code


# ---------------------------------------------------------------------------
# attn_bwd: argument checks
# ---------------------------------------------------------------------------

DQ, DK, DV, DO, LS = 0x600000, 0x700000, 0x800000, 0x900000, 0xA00000


def bwd_args(q=Q, k=K, v=V, o=O, dout=DO, lse=LS, dq=DQ, dk=DK, dv=DV, B=1, H=2, N=128, d=64,
             scale=0.125, dtype=BF16, flags=0):
    from attention_attn_fwd_07_amd import _BwdArgs
    a = _BwdArgs()
    a.q, a.k, a.v, a.o, a.dout, a.lse, a.dq, a.dk, a.dv = q, k, v, o, dout, lse, dq, dk, dv
    a.B, a.H, a.N, a.d, a.scale, a.dtype, a.flags = B, H, N, d, scale, dtype, flags
    a.stream = None
    return a


def call_bwd(lib, ws=W, ws_bytes=1 << 20, **kw):
    from attention_attn_fwd_07_amd import _BwdArgs
    lib.attn_bwd.argtypes = [ctypes.POINTER(_BwdArgs), ctypes.c_void_p, ctypes.c_size_t]
    lib.attn_bwd.restype = ctypes.c_int
    return lib.attn_bwd(ctypes.byref(bwd_args(**kw)), ws, ws_bytes)


def test_bwd_args_struct_matches_the_header(tmp_path):
    import shutil
    import subprocess
    from attention_attn_fwd_07_amd import _BwdArgs
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in _BwdArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "attn_bwd.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(attn_bwd_args_t));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(attn_bwd_args_t, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(_BwdArgs)
    assert got[1:] == [getattr(_BwdArgs, f).offset for f in fields]


def test_bwd_workspace_size(lib):
    lib.attn_bwd_workspace.argtypes = [ctypes.c_int64] * 4
    lib.attn_bwd_workspace.restype = ctypes.c_size_t
    assert lib.attn_bwd_workspace(2, 3, 100, 64) == 2 * 3 * 100 * 8
    assert lib.attn_bwd_workspace(2, 3, 100, 96) == 0
    assert lib.attn_bwd_workspace(0, 3, 100, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), DTYPE), (dict(dtype=5), DTYPE), (dict(d=96), HEAD_DIM),
    (dict(scale=float("nan")), SCALE), (dict(flags=4), FLAGS), (dict(N=-1), SHAPE),
    (dict(dq=None), NULLPTR), (dict(lse=None), NULLPTR), (dict(dout=None), NULLPTR),
    (dict(ws=None), NULLPTR), (dict(dk=DK + 8), ALIGN), (dict(lse=LS + 2), ALIGN),
    (dict(ws=W + 4), ALIGN), (dict(ws_bytes=2 * 128 * 8 - 4), WORKSPACE),
    (dict(dq=Q), ALIAS), (dict(dv=DK + 64), ALIAS), (dict(dk=LS), ALIAS),
    (dict(ws=DV + 128), ALIAS), (dict(ws=LS), ALIAS),
    (dict(N=0), OK), (dict(N=0, dq=None, ws=None), OK),
])
def test_bwd_rejects_before_any_hip_call(lib, kw, code):
    assert call_bwd(lib, **kw) == code


def test_bwd_null_args(lib):
    lib.attn_bwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
    lib.attn_bwd.restype = ctypes.c_int
    assert lib.attn_bwd(None, W, 1 << 20) == NULLPTR


def test_merge_binding_rejects_host_tensors():
    """The merge binding checks the device before any pointer reaches the
    library (a host pointer would reach a kernel)."""
    import torch
    import attention_attn_fwd_07_amd as attn
    o = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        attn.merge([o], [lse])
