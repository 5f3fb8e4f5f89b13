"""Hybrid Top-k + Top-p block-sparse attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libspa.so`` (declared in ``include/spa.h``).
Every step of the computation runs in the library's HIP kernels; this module only
checks tensors, allocates outputs and workspaces with PyTorch, and passes device
pointers and the current HIP stream.  There is no fallback: if the library is missing
or the tensors are not on a ROCm device, the calls raise.

    kv_idx, kv_cnt = build_mask(q, k, blk_q=128, blk_k=64, k_frac=0.05, p=0.9)
    o, lse, o_lo = sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, blk_q=128, blk_k=64,
                                   with_residual=True)
    dq, dk, dv = sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, blk_q=128, blk_k=64,
                                 o_lo=o_lo)
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SpaError", "load_library", "library_path", "build_mask", "sparse_attn_fwd",
    "sparse_attn_bwd", "mask_workspace_bytes", "bwd_workspace_bytes", "status_string",
    "build_mask_noalloc", "NOALLOC_SCRATCH_BYTES",
    "SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libspa.so"
_lib = None

SYMBOLS = ("spa_mask_workspace_bytes", "spa_build_mask", "spa_build_mask_stages",
           "spa_build_mask_noalloc",
           "spa_fwd_workspace_bytes", "spa_sparse_attn_fwd", "spa_sparse_attn_fwd_stages",
           "spa_bwd_workspace_bytes", "spa_sparse_attn_bwd", "spa_sparse_attn_bwd_stages",
           "spa_status_string", "spa_version")
MASK_POOL, MASK_SELECT, MASK_ALL = 1, 2, 3
NOALLOC_SCRATCH_BYTES = 96 << 20  # SPA_NOALLOC_SCRATCH_BYTES
FWD_PREP, FWD_ATTN, FWD_ALL = 1, 2, 3
BWD_PREP, BWD_DQ, BWD_DKDV, BWD_ALL = 1, 2, 4, 7


class SpaError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed ({code}): {text}")
        self.code = code


class _Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("blk_q", ctypes.c_int32), ("blk_k", ctypes.c_int32)]


def library_path() -> str:
    return os.environ.get("SPA_LIBRARY") or os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libspa.so (built in-tree by ``python -m block_sparse_attention_pooled_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with "
                           "`python -m block_sparse_attention_pooled_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
    dp = ctypes.POINTER(_Dims)
    lib.spa_mask_workspace_bytes.argtypes = [dp]
    lib.spa_mask_workspace_bytes.restype = sz
    lib.spa_bwd_workspace_bytes.argtypes = [dp]
    lib.spa_bwd_workspace_bytes.restype = sz
    lib.spa_build_mask.argtypes = [dp, vp, vp, ctypes.c_double, ctypes.c_double,
                                   ctypes.c_double, i32p, i32p, i32p, vp, sz, vp]
    lib.spa_build_mask.restype = ctypes.c_int
    lib.spa_build_mask_stages.argtypes = [dp, vp, vp, ctypes.c_double, ctypes.c_double,
                                          ctypes.c_double, i32p, i32p, i32p, vp, sz,
                                          ctypes.c_uint, vp]
    lib.spa_build_mask_stages.restype = ctypes.c_int
    lib.spa_build_mask_noalloc.argtypes = [dp, vp, vp, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double, i32p, i32p, i32p, vp]
    lib.spa_build_mask_noalloc.restype = ctypes.c_int
    lib.spa_sparse_attn_fwd.argtypes = [dp, vp, vp, vp, i32p, i32p, ctypes.c_double, vp, vp, vp,
                                        vp, sz, vp]
    lib.spa_sparse_attn_fwd_stages.argtypes = [dp, vp, vp, vp, i32p, i32p, ctypes.c_double, vp,
                                               vp, vp, vp, sz, ctypes.c_uint, vp]
    lib.spa_sparse_attn_fwd_stages.restype = ctypes.c_int
    lib.spa_fwd_workspace_bytes.argtypes = [dp]
    lib.spa_fwd_workspace_bytes.restype = sz
    lib.spa_sparse_attn_fwd.restype = ctypes.c_int
    lib.spa_sparse_attn_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i32p, i32p,
                                        ctypes.c_double, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    lib.spa_sparse_attn_bwd.restype = ctypes.c_int
    lib.spa_sparse_attn_bwd_stages.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i32p, i32p,
                                               ctypes.c_double, vp, vp, vp, ctypes.c_int, vp, sz,
                                               ctypes.c_uint, vp]
    lib.spa_sparse_attn_bwd_stages.restype = ctypes.c_int
    lib.spa_status_string.argtypes = [ctypes.c_int]
    lib.spa_status_string.restype = ctypes.c_char_p
    lib.spa_version.argtypes = []
    lib.spa_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().spa_status_string(code).decode()


def _dims(shape, blk_q: int, blk_k: int) -> _Dims:
    B, H, N, d = (int(x) for x in shape)
    return _Dims(B, H, N, d, int(blk_q), int(blk_k))


def mask_workspace_bytes(shape, blk_q: int, blk_k: int = 64) -> int:
    return int(load_library().spa_mask_workspace_bytes(ctypes.byref(_dims(shape, blk_q, blk_k))))


def fwd_workspace_bytes(shape, blk_q: int, blk_k: int = 64) -> int:
    return int(load_library().spa_fwd_workspace_bytes(ctypes.byref(_dims(shape, blk_q, blk_k))))


def bwd_workspace_bytes(shape, blk_q: int, blk_k: int = 64) -> int:
    return int(load_library().spa_bwd_workspace_bytes(ctypes.byref(_dims(shape, blk_q, blk_k))))


def _check(fn: str, rc: int):
    if rc != 0:
        raise SpaError(fn, rc, status_string(rc))


def _torch():
    import torch
    return torch


def _dev_tensor(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor on a ROCm (HIP) device")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out_tensor(t, dtype, shape, name, device):
    """A caller-supplied output: the dtype, shape and device the kernels write, contiguous."""
    _dev_tensor(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _workspace(ws, need: int, device, name: str):
    """(tensor, byte count) of a workspace: allocated here when not given, else checked to
    be a contiguous device tensor of at least `need` bytes."""
    torch = _torch()
    if ws is None:
        return torch.empty(max(1, need), dtype=torch.uint8, device=device), max(1, need)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"{name} holds {nbytes} bytes; {need} are needed")
    return ws, nbytes


def _stream(dev):
    return ctypes.c_void_p(_torch().cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def n_blocks(N: int, blk: int) -> int:
    return -(-N // blk)


def build_mask(q, k, blk_q: int = 128, blk_k: int = 64, k_frac: float = 0.05, p: float = 0.9,
               pooled_scale: float | None = None, rule_len: bool = False, out=None,
               workspace=None, stages: int = MASK_ALL):
    """Hybrid Top-k + Top-p block mask.  Returns (kv_idx, kv_cnt[, rule_len]).

    kv_idx: int32 [B, H, Nqb, Nkb], ascending kept key blocks in the first kv_cnt entries
    of each row; kv_cnt: int32 [B, H, Nqb]; rule_len: int32 [B, H, Nqb, 2] = (Lk, Lp).
    """
    torch = _torch()
    lib = load_library()
    _dev_tensor(q, torch.bfloat16, "q")
    _dev_tensor(k, torch.bfloat16, "k")
    if q.shape != k.shape or q.dim() != 4:
        raise ValueError("q and k must both be [B, H, N, d]")
    B, H, N, d = q.shape
    nqb, nkb = n_blocks(N, blk_q), n_blocks(N, blk_k)
    dims = _dims(q.shape, blk_q, blk_k)
    if k.device != q.device:
        raise ValueError("q and k must be on the same device")
    if out is None:
        kv_idx = torch.empty((B, H, nqb, nkb), dtype=torch.int32, device=q.device)
        kv_cnt = torch.empty((B, H, nqb), dtype=torch.int32, device=q.device)
        rl = torch.empty((B, H, nqb, 2), dtype=torch.int32, device=q.device) if rule_len else None
    else:
        kv_idx, kv_cnt, rl = out
        _out_tensor(kv_idx, torch.int32, (B, H, nqb, nkb), "kv_idx", q.device)
        _out_tensor(kv_cnt, torch.int32, (B, H, nqb), "kv_cnt", q.device)
        if rule_len and rl is None:
            raise ValueError("rule_len=True needs a rule_len tensor in out")
        if rl is not None:
            _out_tensor(rl, torch.int32, (B, H, nqb, 2), "rule_len", q.device)
    ws, wsn = _workspace(workspace, int(lib.spa_mask_workspace_bytes(ctypes.byref(dims))),
                         q.device, "workspace")
    rc = lib.spa_build_mask_stages(ctypes.byref(dims), _ptr(q), _ptr(k), float(k_frac),
                                   float(p), float(pooled_scale or 0.0), _ptr(kv_idx),
                                   _ptr(kv_cnt), _ptr(rl), _ptr(ws), wsn, int(stages),
                                   _stream(q.device))
    _check("spa_build_mask", rc)
    return (kv_idx, kv_cnt, rl) if rule_len else (kv_idx, kv_cnt)


def build_mask_noalloc(q, k, kv_idx, kv_cnt, blk_q: int = 128, blk_k: int = 64,
                       k_frac: float = 0.05, p: float = 0.9, pooled_scale: float | None = None,
                       rule_len=None):
    """build_mask into caller-given outputs through spa_build_mask_noalloc: no workspace,
    no allocation (the pooled means use the library's fixed device scratch of
    NOALLOC_SCRATCH_BYTES).  kv_idx int32 [B, H, Nqb, Nkb], kv_cnt int32 [B, H, Nqb] and the
    optional rule_len int32 [B, H, Nqb, 2] are written in place.  Calls that overlap on one
    GPU share the scratch and race."""
    torch = _torch()
    lib = load_library()
    _dev_tensor(q, torch.bfloat16, "q")
    _dev_tensor(k, torch.bfloat16, "k")
    if q.shape != k.shape or q.dim() != 4:
        raise ValueError("q and k must both be [B, H, N, d]")
    if k.device != q.device:
        raise ValueError("q and k must be on the same device")
    B, H, N, d = q.shape
    nqb, nkb = n_blocks(N, blk_q), n_blocks(N, blk_k)
    _out_tensor(kv_idx, torch.int32, (B, H, nqb, nkb), "kv_idx", q.device)
    _out_tensor(kv_cnt, torch.int32, (B, H, nqb), "kv_cnt", q.device)
    if rule_len is not None:
        _out_tensor(rule_len, torch.int32, (B, H, nqb, 2), "rule_len", q.device)
    dims = _dims(q.shape, blk_q, blk_k)
    rc = lib.spa_build_mask_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), float(k_frac),
                                    float(p), float(pooled_scale or 0.0), _ptr(kv_idx),
                                    _ptr(kv_cnt), _ptr(rule_len), _stream(q.device))
    _check("spa_build_mask_noalloc", rc)


def sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, blk_q: int = 128, blk_k: int = 64,
                    scale: float | None = None, with_residual: bool = False, out=None,
                    workspace=None, stages: int = FWD_ALL):
    """Block-sparse attention forward.

    Returns (o bf16 [B,H,N,d], lse fp32 [B,H,N]), or (o, lse, o_lo) with
    ``with_residual=True``: o_lo is the bf16 rounding residual of O that the backward
    pass uses for D = <dO, O>.  The residual mode needs a device workspace of
    fwd_workspace_bytes() (allocated here when not given).  ``stages`` selects FWD_PREP
    (the fp16 copy of V into the workspace; it reads V only) and/or FWD_ATTN, which with
    the residual reads what FWD_PREP wrote into the same workspace.
    """
    torch = _torch()
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, torch.bfloat16, n)
    _dev_tensor(kv_idx, torch.int32, "kv_idx")
    _dev_tensor(kv_cnt, torch.int32, "kv_cnt")
    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError("q, k, v must all be [B, H, N, d]")
    B, H, N, d = q.shape
    nqb, nkb = n_blocks(N, blk_q), n_blocks(N, blk_k)
    if tuple(kv_idx.shape) != (B, H, nqb, nkb) or tuple(kv_cnt.shape) != (B, H, nqb):
        raise ValueError("kv_idx / kv_cnt shapes do not match q and the block sizes")
    for t, n in ((k, "k"), (v, "v"), (kv_idx, "kv_idx"), (kv_cnt, "kv_cnt")):
        if t.device != q.device:
            raise ValueError(f"{n} must be on {q.device}")
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        o_lo = torch.empty_like(q) if with_residual else None
    else:
        o, lse, o_lo = out
        _out_tensor(o, torch.bfloat16, q.shape, "o", q.device)
        _out_tensor(lse, torch.float32, (B, H, N), "lse", q.device)
        if with_residual and o_lo is None:
            raise ValueError("with_residual=True needs an o_lo tensor in out")
        if o_lo is not None:
            _out_tensor(o_lo, torch.bfloat16, q.shape, "o_lo", q.device)
    dims = _dims(q.shape, blk_q, blk_k)
    ws, wsn = None, 0
    if o_lo is not None:
        ws, wsn = _workspace(workspace, int(lib.spa_fwd_workspace_bytes(ctypes.byref(dims))),
                             q.device, "workspace")
    rc = lib.spa_sparse_attn_fwd_stages(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(kv_idx), _ptr(kv_cnt), float(scale or 0.0), _ptr(o),
                                        _ptr(o_lo), _ptr(lse), _ptr(ws), wsn, int(stages),
                                        _stream(q.device))
    _check("spa_sparse_attn_fwd", rc)
    return (o, lse, o_lo) if with_residual else (o, lse)


def sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, blk_q: int = 128, blk_k: int = 64,
                    scale: float | None = None, o_lo=None, grad_dtype=None, out=None,
                    workspace=None, stages: int = BWD_ALL):
    """Block-sparse attention backward.  Returns (dq, dk, dv), fp32 unless grad_dtype=bf16.

    Pass the forward's ``o_lo`` residual for full accuracy of D = <dO, O>.  Tensors given
    in ``out`` must have the gradient dtype, the shape of q and be contiguous on q's device.
    """
    torch = _torch()
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _dev_tensor(t, torch.bfloat16, n)
    if o_lo is not None:
        _dev_tensor(o_lo, torch.bfloat16, "o_lo")
        if o_lo.shape != o.shape:
            raise ValueError("o_lo must have the shape of o")
    _dev_tensor(lse, torch.float32, "lse")
    _dev_tensor(kv_idx, torch.int32, "kv_idx")
    _dev_tensor(kv_cnt, torch.int32, "kv_cnt")
    if not (q.shape == k.shape == v.shape == o.shape == do.shape) or q.dim() != 4:
        raise ValueError("q, k, v, o, do must all be [B, H, N, d]")
    B, H, N, d = q.shape
    nqb, nkb = n_blocks(N, blk_q), n_blocks(N, blk_k)
    if tuple(kv_idx.shape) != (B, H, nqb, nkb) or tuple(kv_cnt.shape) != (B, H, nqb):
        raise ValueError("kv_idx / kv_cnt shapes do not match q and the block sizes")
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    gdt = torch.float32 if grad_dtype in (None, torch.float32) else grad_dtype
    if gdt not in (torch.float32, torch.bfloat16):
        raise ValueError("grad_dtype must be float32 or bfloat16")
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do"), (lse, "lse"), (kv_idx, "kv_idx"),
                 (kv_cnt, "kv_cnt"), (o_lo, "o_lo")):
        if t is not None and t.device != q.device:
            raise ValueError(f"{n} must be on {q.device}")
    if out is None:
        dq, dk, dv = (torch.empty(q.shape, dtype=gdt, device=q.device) for _ in range(3))
    else:
        dq, dk, dv = out
        for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            _out_tensor(t, gdt, q.shape, n, q.device)
    dims = _dims(q.shape, blk_q, blk_k)
    ws, wsn = _workspace(workspace, int(lib.spa_bwd_workspace_bytes(ctypes.byref(dims))),
                         q.device, "workspace")
    rc = lib.spa_sparse_attn_bwd_stages(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_lo), _ptr(do), _ptr(lse),
        _ptr(kv_idx), _ptr(kv_cnt), float(scale or 0.0), _ptr(dq), _ptr(dk), _ptr(dv),
        1 if gdt == torch.bfloat16 else 0, _ptr(ws), wsn, int(stages), _stream(q.device))
    _check("spa_sparse_attn_bwd", rc)
    return dq, dk, dv
