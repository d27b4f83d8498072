"""attention_attn_fwd_07_amd - fused attention forward on MI355X (gfx950).

A thin ctypes binding over ``libattn_fwd.so`` (declared in
``include/attn_fwd.h``).  It only marshals arguments: torch supplies device
memory and the current HIP stream, every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library is missing, or no
GPU is present, calls raise.

    o, lse = fwd(q, k, v)                  # allocate outputs, scale = 1/sqrt(d)
    attn_fwd(q, k, v, o, lse, scale)       # caller-owned outputs, async launch
    p = plan(q, k, v, o, lse, scale); p()  # checked once, then relaunched cheaply
    o, lse = fwd_splitkv(q, k, v, splits=8)  # keys split over 8 blocks, then merged
    attn_fwd_splitkv_static(q, k, v, o, lse, scale, 4)  # no workspace, no allocation
    dq, dk, dv = bwd(q, k, v, o, lse, do)    # gradients (include/attn_bwd.h)
    o = attention(q, k, v)                 # with autograd: o.backward(do) runs attn_bwd
    o, lse = merge([o1, o2], [lse1, lse2])   # results over two key shards -> over both

Tensors are ``[B, H, N, d]`` fp32/fp16/bf16 with d in {64, 128}; k and v may
have their own number of rows Nk (``[B, H, Nk, d]``: a few queries against a
long key/value history), q, o and lse keep N.  The head dimension must be
contiguous, the other three dimensions may have any strides that are multiples
of 8 elements (so a ``[B, N, H, d]`` tensor viewed with ``.transpose(1, 2)`` is
accepted without a copy).  ``lse`` is ``[B, H, N]`` fp32 contiguous (or None).
``causal=True`` (only with Nk = N) restricts query row i to keys 0..i.
Argument errors raise ValueError, mirroring a wrapper that checks device,
shape, dtype and layout before it launches anything (page 2 "Triton
programming template", Python wrapper).
"""
from __future__ import annotations

import ctypes
import math
import os

from .build import LIB

__all__ = ["attn_fwd", "fwd", "plan", "Plan", "attn_strerror", "attn_version", "library_path",
           "AttnError", "ATTN_CAUSAL", "splitkv_workspace_size", "fwd_splitkv", "attn_bwd",
           "bwd", "bwd_workspace_size", "attn_fwd_splitkv_static", "STATIC_WORKSPACE_BYTES",
           "attention", "merge"]

STATIC_WORKSPACE_BYTES = 64 << 20  # ATTN_STATIC_WORKSPACE_BYTES of include/attn_fwd.h

ATTN_OK = 0
ATTN_ERR_HIP = -8
ATTN_CAUSAL = 1


class _BwdArgs(ctypes.Structure):
    """attn_bwd_args_t of include/attn_bwd.h."""

    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64), ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
                ("flags", ctypes.c_uint), ("stream", ctypes.c_void_p)]


class _Args(ctypes.Structure):
    """attn_fwd_args_t of include/attn_fwd.h."""

    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64), ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
                ("flags", ctypes.c_uint),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
                ("stream", ctypes.c_void_p), ("Nk", ctypes.c_int64)]


class AttnError(ValueError):
    """An argument error reported by the library (a negative return code)."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"attn_fwd error {code}: {msg}")
        self.code = code


_lib = None


def library_path() -> str:
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise ImportError(
            f"{LIB} is not built; run `python -m attention_attn_fwd_07_amd.build` "
            "(the HIP library is required: there is no CPU fallback)")
    lib = ctypes.CDLL(LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                             ctypes.c_int, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_ex.argtypes = [ctypes.POINTER(_Args)]
    lib.attn_fwd_ex.restype = ctypes.c_int
    lib.attn_fwd_splitkv.argtypes = [ctypes.POINTER(_Args), ctypes.c_int, vp, ctypes.c_size_t]
    lib.attn_fwd_splitkv.restype = ctypes.c_int
    lib.attn_fwd_splitkv_static.argtypes = [ctypes.POINTER(_Args), ctypes.c_int]
    lib.attn_fwd_splitkv_static.restype = ctypes.c_int
    lib.attn_fwd_splitkv_workspace.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.attn_fwd_splitkv_workspace.restype = ctypes.c_size_t
    lib.attn_fwd_splitkv_workspace_ex.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int]
    lib.attn_fwd_splitkv_workspace_ex.restype = ctypes.c_size_t
    lib.attn_fwd_merge.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int, vp, vp,
                                   i64, i64, i64, i64, ctypes.c_int, vp]
    lib.attn_fwd_merge.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [ctypes.POINTER(_BwdArgs), vp, ctypes.c_size_t]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_workspace.argtypes = [i64, i64, i64, i64]
    lib.attn_bwd_workspace.restype = ctypes.c_size_t
    lib.attn_strerror.argtypes = [ctypes.c_int]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_int
    _lib = lib
    return lib


def attn_strerror(code: int) -> str:
    return _load().attn_strerror(int(code)).decode()


def attn_version() -> int:
    return int(_load().attn_version())


def _torch():
    import torch
    return torch


def _dtype_codes():
    torch = _torch()
    return {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def _check(q, k, v, o, lse):
    torch = _torch()
    codes = _dtype_codes()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d]")
        if t.numel() > 0 and t.stride(3) != 1 and t.shape[3] > 1:
            raise ValueError(f"{name}: the head dimension must be contiguous")
    # q and o: [B, H, N, d]; k and v: [B, H, Nk, d] with Nk >= 1 keys when N > 0
    if not (q.shape == o.shape and k.shape == v.shape and q.shape[:2] == k.shape[:2]
            and q.shape[3] == k.shape[3]):
        raise ValueError(f"shape mismatch: q{tuple(q.shape)} k{tuple(k.shape)} "
                         f"v{tuple(v.shape)} o{tuple(o.shape)}")
    if k.shape[2] == 0 and q.numel() > 0:
        raise ValueError("k and v have no rows: a softmax over no keys is undefined")
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise ValueError("q, k, v and o must share one dtype")
    if q.dtype not in codes:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if not (q.device == k.device == v.device == o.device):
        raise ValueError("q, k, v and o must be on the same device")
    if lse is not None:
        if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32:
            raise ValueError("lse must be a float32 tensor or None")
        if lse.device != q.device or not lse.is_contiguous():
            raise ValueError("lse must be contiguous and on q's device")
        if tuple(lse.shape) != tuple(q.shape[:3]):
            raise ValueError(f"lse must have shape {tuple(q.shape[:3])}")
    return codes[q.dtype]


def _raise_for(rc: int) -> None:
    if rc == ATTN_ERR_HIP:
        raise RuntimeError(f"attn_fwd: {attn_strerror(rc)}")
    if rc != ATTN_OK:
        raise AttnError(rc, attn_strerror(rc))


def _strides(t):
    """(batch, head, row) element strides, or zeros for a contiguous tensor.

    All-zero strides are the C ABI's mark of a contiguous tensor, so a
    non-contiguous tensor whose three leading strides are all zero (one row
    broadcast to every (b, h, n), as ``t[:1, :1, :1].expand(...)`` makes) has
    no stride triple of its own; ``_unbroadcast`` handles it before this."""
    if t.is_contiguous():
        return (0, 0, 0)
    st = tuple(int(x) for x in t.stride()[:3])
    if st == (0, 0, 0):
        raise ValueError("a tensor broadcast from a single row has no stride triple; "
                         "pass it through _unbroadcast (inputs) or use a real output")
    return st


def _unbroadcast(t, name: str, output: bool = False):
    """An input whose batch, head and row strides are all zero (one row
    broadcast over the whole [B, H, N, d] shape) is copied to a contiguous
    tensor with the same values; an output of that form cannot hold distinct
    rows and is rejected."""
    if t.numel() == 0 or t.is_contiguous() or tuple(t.stride()[:3]) != (0, 0, 0):
        return t
    if output:
        raise ValueError(f"{name}: an output broadcast from a single row cannot hold the result")
    return t.contiguous()


class Plan:
    """One checked ``attn_fwd_ex`` call whose arguments are marshalled once.

    The tensors are validated when the plan is made; each call then only
    passes the stored pointers, sizes and stream to the library (which still
    validates them), so repeated launches cost little host time.  The caller
    keeps the tensors alive and unchanged in shape while the plan is used.
    """

    def __init__(self, q, k, v, o, lse, scale: float, stream=None, causal: bool = False,
                 splits: int = 0, workspace=None, static_workspace: bool = False):
        torch = _torch()
        code_dtype = _check(q, k, v, o, lse)
        q, k, v = (_unbroadcast(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v")))
        _unbroadcast(o, "o", output=True)
        B, H, N, d = (int(x) for x in q.shape)
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        elif hasattr(stream, "cuda_stream"):
            stream = stream.cuda_stream
        self.device = q.device
        lib = _load()
        a = _Args()
        a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
        a.lse = lse.data_ptr() if lse is not None else None
        a.B, a.H, a.N, a.d = B, H, N, d
        a.Nk = int(k.shape[2])
        a.scale = float(scale)
        a.dtype = code_dtype
        a.flags = ATTN_CAUSAL if causal else 0
        a.q_stride[:] = _strides(q)
        a.k_stride[:] = _strides(k)
        a.v_stride[:] = _strides(v)
        a.o_stride[:] = _strides(o)
        a.stream = stream
        self._args = a
        self._ref = ctypes.byref(a)
        if splits and static_workspace:
            if workspace is not None:
                raise ValueError("the static split-KV path takes no workspace")
            fn = lib.attn_fwd_splitkv_static
            self._call = lambda: fn(self._ref, int(splits))
        elif splits:
            if workspace is None:
                raise ValueError("the split-KV path needs a workspace tensor")
            if workspace.device != q.device or not workspace.is_contiguous():
                raise ValueError("workspace must be contiguous and on q's device")
            nbytes = workspace.numel() * workspace.element_size()
            fn, ws = lib.attn_fwd_splitkv, ctypes.c_void_p(workspace.data_ptr())
            self._call = lambda: fn(self._ref, int(splits), ws, nbytes)
        else:
            fn = lib.attn_fwd_ex
            self._call = lambda: fn(self._ref)
        self._tensors = (q, k, v, o, lse, workspace)  # keep the storage alive

    def __call__(self) -> None:
        rc = self._call()
        if rc != ATTN_OK:
            _raise_for(rc)


def plan(q, k, v, o, lse, scale: float, stream=None, causal: bool = False, splits: int = 0,
         workspace=None) -> Plan:
    """Check the arguments of ``attn_fwd_ex`` (or, with ``splits``, of
    ``attn_fwd_splitkv``) once and return a relaunchable call.

    q's device must be the current device whenever the plan is called."""
    return Plan(q, k, v, o, lse, scale, stream, causal, splits, workspace)


def splitkv_workspace_size(B: int, H: int, N: int, d: int, splits: int,
                           Nk: int | None = None) -> int:
    """Bytes of workspace ``attn_fwd_splitkv`` needs for N query rows and Nk
    key rows per head (Nk defaults to N; 0 for empty sizes)."""
    if Nk is None:
        return int(_load().attn_fwd_splitkv_workspace(B, H, N, d, splits))
    return int(_load().attn_fwd_splitkv_workspace_ex(B, H, N, Nk, d, splits))


def fwd_splitkv(q, k, v, scale: float | None = None, splits: int = 4, workspace=None,
                return_lse: bool = True):
    """``fwd`` through the split-KV path: each head's keys split into up to
    ``splits`` ranges handled by separate blocks, the partial results merged
    by a second kernel.  Allocates the workspace if none is given."""
    torch = _torch()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    B, H, N, d = (int(x) for x in q.shape)
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = (torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
           if return_lse else None)
    if workspace is None:
        nbytes = splitkv_workspace_size(B, H, N, d, splits, int(k.shape[2]))
        workspace = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device=q.device)
    p = Plan(q, k, v, o, lse, scale, None, False, splits, workspace)
    if torch.cuda.current_device() == p.device.index:
        p()
    else:
        with torch.cuda.device(p.device):
            p()
    return o, lse


def attn_fwd_splitkv_static(q, k, v, o, lse, scale: float, splits: int, stream=None) -> None:
    """``attn_fwd_splitkv`` into the caller's ``o`` and ``lse`` with the
    library's own static device workspace (ATTN_STATIC_WORKSPACE_BYTES): the
    library allocates nothing.  Calls on one device share that workspace, so
    overlapping calls (different streams) race; order them on one stream."""
    torch = _torch()
    p = Plan(q, k, v, o, lse, scale, stream, False, splits, None, static_workspace=True)
    if torch.cuda.current_device() == p.device.index:
        p()
    else:
        with torch.cuda.device(p.device):
            p()


def attn_fwd(q, k, v, o, lse, scale: float, stream=None, causal: bool = False) -> None:
    """O = softmax(scale * Q K^T) V into ``o`` (and the log-sum-exp into ``lse``).

    Asynchronous on ``stream`` (default: torch's current stream of q's device).
    ``causal``: query row i attends keys 0..i only.
    """
    torch = _torch()
    p = Plan(q, k, v, o, lse, scale, stream, causal)
    if torch.cuda.current_device() == p.device.index:
        p()
    else:
        with torch.cuda.device(p.device):
            p()


def fwd(q, k, v, scale: float | None = None, return_lse: bool = True, causal: bool = False):
    """Allocate O (and lse) and run ``attn_fwd``; scale defaults to 1/sqrt(d).

    O is allocated contiguous [B, H, N, d] whatever q's strides."""
    torch = _torch()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = (torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
           if return_lse else None)
    attn_fwd(q, k, v, o, lse, scale, causal=causal)
    return o, lse


def merge(o_parts, lse_parts, o=None, lse=None, stream=None):
    """``attn_fwd_merge``: the results over disjoint key sets (each an O of shape
    [B, H, N, d] and its fp32 lse [B, H, N], as ``fwd`` returns them for one
    shard of the keys) combined into the result over all the keys.  Allocates
    ``o`` and ``lse`` if not given; returns (o, lse)."""
    torch = _torch()
    codes = _dtype_codes()
    if len(o_parts) != len(lse_parts) or not o_parts:
        raise ValueError("o_parts and lse_parts must be non-empty and of equal length")
    o0 = o_parts[0]
    if not isinstance(o0, torch.Tensor) or o0.dtype not in codes or o0.dim() != 4:
        raise ValueError("each part's O must be a 4-D float32/float16/bfloat16 tensor")
    if o0.device.type != "cuda":
        raise ValueError("the parts must be GPU tensors")
    for x, l in zip(o_parts, lse_parts):
        if (x.shape != o0.shape or x.dtype != o0.dtype or x.device != o0.device
                or not x.is_contiguous()):
            raise ValueError("every part's O must be contiguous with the first one's shape, "
                             "dtype and device")
        if (l is None or l.dtype != torch.float32 or tuple(l.shape) != tuple(o0.shape[:3])
                or l.device != o0.device or not l.is_contiguous()):
            raise ValueError("every part needs a contiguous float32 lse of shape [B, H, N]")
    if o is None:
        o = torch.empty_like(o0)
    if lse is None:
        lse = torch.empty(o0.shape[:3], dtype=torch.float32, device=o0.device)
    if (not isinstance(o, torch.Tensor) or o.shape != o0.shape or o.dtype != o0.dtype
            or o.device != o0.device or not o.is_contiguous()):
        raise ValueError("o must be contiguous with the parts' shape, dtype and device")
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32
            or tuple(lse.shape) != tuple(o0.shape[:3]) or lse.device != o0.device
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on the parts' device")
    if stream is None:
        stream = torch.cuda.current_stream(o0.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    n = len(o_parts)
    optrs = (ctypes.c_void_p * n)(*[x.data_ptr() for x in o_parts])
    lptrs = (ctypes.c_void_p * n)(*[x.data_ptr() for x in lse_parts])
    B, H, N, d = (int(x) for x in o0.shape)
    with torch.cuda.device(o0.device):
        rc = _load().attn_fwd_merge(optrs, lptrs, n, o.data_ptr(), lse.data_ptr(), B, H, N, d,
                                    codes[o0.dtype], stream)
    if rc != ATTN_OK:
        _raise_for(rc)
    return o, lse


def bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    """Bytes of workspace ``attn_bwd`` needs (0 for empty sizes)."""
    return int(_load().attn_bwd_workspace(B, H, N, d))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale: float, workspace, stream=None,
             causal: bool = False) -> None:
    """dQ, dK, dV of O = softmax(scale Q K^T) V into the caller's ``dq``, ``dk``,
    ``dv`` (contiguous [B, H, N, d], q's dtype), given the forward's ``o``
    and ``lse`` and the upstream gradient ``dout``.  Asynchronous on ``stream``."""
    torch = _torch()
    code = _check(q, k, v, o, lse)
    if k.shape != q.shape:
        raise ValueError("the backward is for self-attention: k and v need q's shape")
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if not isinstance(t, torch.Tensor) or t.device != q.device:
            raise ValueError(f"{name} must be a tensor on q's device")
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q's shape and dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous for the backward")
    if lse is None:
        raise ValueError("the backward needs the forward's lse")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    a = _BwdArgs()
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    a.dout, a.lse = dout.data_ptr(), lse.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.B, a.H, a.N, a.d = (int(x) for x in q.shape)
    a.scale = float(scale)
    a.dtype = code
    a.flags = ATTN_CAUSAL if causal else 0
    a.stream = stream
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    wptr = workspace.data_ptr() if workspace is not None else None
    with torch.cuda.device(q.device):
        rc = _load().attn_bwd(ctypes.byref(a), ctypes.c_void_p(wptr), nbytes)
    if rc != ATTN_OK:
        _raise_for(rc)


def bwd(q, k, v, o, lse, dout, scale: float | None = None, causal: bool = False):
    """Allocate dq, dk, dv and the workspace, run ``attn_bwd``, return the grads."""
    torch = _torch()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    B, H, N, d = (int(x) for x in q.shape)
    nbytes = bwd_workspace_size(B, H, N, d)
    ws = torch.empty(max(4, nbytes) // 4, dtype=torch.float32, device=q.device)
    attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale, ws, causal=causal)
    return dq, dk, dv


_ATTENTION_FN = None


def _attention_fn():
    """The autograd Function behind ``attention`` (made on first use, since
    torch is imported lazily)."""
    global _ATTENTION_FN
    if _ATTENTION_FN is None:
        torch = _torch()

        class AttentionFn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, scale, causal):
                o, lse = fwd(q, k, v, scale, True, causal)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.scale, ctx.causal = scale, causal
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), ctx.scale, ctx.causal)
                return dq, dk, dv, None, None

        _ATTENTION_FN = AttentionFn
    return _ATTENTION_FN


def attention(q, k, v, scale: float | None = None, causal: bool = False):
    """O = softmax(scale Q K^T) V as a differentiable torch op: the forward runs
    ``attn_fwd`` and keeps q, k, v, O and the log-sum-exp; the backward runs
    ``attn_bwd`` on them (page 3 "OpenAI Triton from introduction to model
    practice", section 6: the autograd wrapper saves q, k, v, o and lse for the
    backward).  Gradients need contiguous q, k, v of one length."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _attention_fn().apply(q, k, v, float(scale), bool(causal))
