"""Python binding of libfa (exact tiled attention for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfa.so``.  PyTorch supplies device memory and the current
stream.  If the library has not been built this module raises on first use;
there is no fallback path.

    o, lse = forward(q, k, v, scale, causal=False, blockmask=None)
    dq, dk, dv = backward(q, k, v, o, do, lse, scale, causal=False, blockmask=None)

Tensors are [B, H, N, d] bfloat16, contiguous, on one GPU; ``blockmask`` is
a uint8 [nb, nb] tensor on the same GPU (nb = ceil(N / mask_block)).
"""

from __future__ import annotations

import ctypes
import math
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "fa.h")

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_UNSUPPORTED = 3
FA_ERR_WORKSPACE = 4
FA_ERR_HIP = 5
FA_ERR_SCRATCH = 6
NOALLOC_MAX_ROWS = 4194304   # FA_NOALLOC_MAX_ROWS: B*H*N limit of fa_bwd_noalloc

_lib = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_u64, _u32 = ctypes.c_uint64, ctypes.c_uint32
_SIGNATURES = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i, _vp, _vp, _vp]),
    "fa_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i,
                    _vp, _vp, _vp, _vp, _sz, _vp]),
    "fa_bwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i,
                            _vp, _vp, _vp, _vp]),
    "fa_bwd_dsum": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "fa_bwd_dkdv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i,
                         _vp, _vp, _vp]),
    "fa_bwd_dq": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i,
                       _vp, _vp]),
    "fa_bwd_dq_dsum": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i,
                            _vp, _vp, _vp]),
    "fa_fwd_dropout": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i, _f, _u64, _u32,
                            _vp, _vp, _vp]),
    "fa_bwd_dropout": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i,
                            _f, _u64, _u32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "fa_dropout_keep_mask": (_i, [_i, _i, _i, _f, _u64, _u32, _vp, _vp]),
    "fa_fwd_nqk": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _i, _vp, _vp, _vp]),
    "fa_bwd_nqk": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _i,
                        _vp, _vp, _vp, _vp, _sz, _vp]),
    "fa_fwd_splitkv": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _i, _i, _vp, _sz,
                            _vp, _vp, _vp]),
    "fa_fwd_splitkv_num_splits": (_i, [_i, _i, _i, _i, _i]),
    "fa_fwd_splitkv_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "fa_fwd_fp8": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _f, _f, _f, _i, _vp, _i, _vp, _vp,
                        _vp]),
    "fa_strerror": (ctypes.c_char_p, [_i]),
}


class LibfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def load_library(path: str = LIB_PATH):
    """Load libfa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libfa.so not found at {path}; build it with `python -m exact_io_aware_62_amd.build`")
    # torch ships its own HIP runtime, with the same soname as the system's but
    # linked by file name.  Loaded first, it satisfies libfa's dependency, so
    # libfa and torch share one runtime and torch's streams are valid in libfa;
    # loaded after libfa, it would bring a second runtime and launches on
    # torch's streams would fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions include/fa.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)


def strerror(status: int) -> str:
    return load_library().fa_strerror(int(status)).decode()


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, N, d))


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch  # local: the C ABI itself needs no torch
    return torch


def _check(t, name, dtype, shape=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (BHND)")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _mask_args(blockmask, N, mask_block, device, Nk=None):
    torch = _torch()
    if blockmask is None:
        return None, 0
    nb = -(-N // mask_block)
    nbk = nb if Nk is None else -(-Nk // mask_block)
    _check(blockmask, "blockmask", torch.uint8, (nb, nbk), device)
    return blockmask.data_ptr(), mask_block


def _stream_ptr(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def forward(q, k, v, scale: float | None = None, causal: bool = False, blockmask=None,
            mask_block: int = 128, out=None, lse=None, dropout_p: float = 0.0, seed: int = 0,
            offset: int = 0):
    """O, LSE = attention forward.  Returns (o [B,H,N,d] bf16, lse [B,H,N] fp32).

    k and v may have another sequence length Nk than q (fa_fwd_nqk; the causal
    mask is then aligned bottom-right).  dropout_p > 0 runs fa_fwd_dropout with
    that (p, seed, offset); pass the same three to ``backward``."""
    torch = _torch()
    _check(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    dev = q.device
    if k.dim() != 4:
        raise ValueError("k must be [B, H, Nk, d]")
    Nk = k.shape[2]
    kshape = (B, H, Nk, d)
    _check(k, "k", torch.bfloat16, kshape, dev)
    _check(v, "v", torch.bfloat16, kshape, dev)
    if Nk != N and dropout_p:
        raise ValueError("dropout is supported with equal query and key lengths only")
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, q.shape, dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    else:
        _check(lse, "lse", torch.float32, (B, H, N), dev)
    bm_ptr, mb = _mask_args(blockmask, N, mask_block, dev, Nk)
    if dropout_p:
        rc = load_library().fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d,
                                           scale, int(bool(causal)), bm_ptr, mb,
                                           float(dropout_p), int(seed), int(offset),
                                           out.data_ptr(), lse.data_ptr(), _stream_ptr(dev))
        if rc != FA_OK:
            raise LibfaError(rc, "fa_fwd_dropout")
        return out, lse
    if Nk != N:
        rc = load_library().fa_fwd_nqk(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, Nk, d,
                                       scale, int(bool(causal)), bm_ptr, mb, out.data_ptr(),
                                       lse.data_ptr(), _stream_ptr(dev))
        if rc != FA_OK:
            raise LibfaError(rc, "fa_fwd_nqk")
        return out, lse
    rc = load_library().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d, scale,
                               int(bool(causal)), bm_ptr, mb, out.data_ptr(), lse.data_ptr(),
                               _stream_ptr(dev))
    if rc != FA_OK:
        raise LibfaError(rc, "fa_fwd")
    return out, lse


def backward(q, k, v, o, do, lse, scale: float | None = None, causal: bool = False,
             blockmask=None, mask_block: int = 128, workspace=None, dq=None, dk=None, dv=None,
             dropout_p: float = 0.0, seed: int = 0, offset: int = 0):
    """dQ, dK, dV of sum(dO * O).  Returns (dq [B,H,N,d], dk, dv [B,H,Nk,d]) bf16.

    k and v may have another length Nk than q (fa_bwd_nqk).  dropout_p > 0 runs
    fa_bwd_dropout (the forward must have used the same dropout_p, seed and
    offset)."""
    torch = _torch()
    _check(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    dev = q.device
    if k.dim() != 4:
        raise ValueError("k must be [B, H, Nk, d]")
    Nk = k.shape[2]
    kshape = (B, H, Nk, d)
    for name, t, shape in (("k", k, kshape), ("v", v, kshape), ("o", o, q.shape),
                           ("do", do, q.shape)):
        _check(t, name, torch.bfloat16, shape, dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    if Nk != N and dropout_p:
        raise ValueError("dropout is supported with equal query and key lengths only")
    scale = default_scale(d) if scale is None else float(scale)
    outs = []
    for name, t, shape in (("dq", dq, q.shape), ("dk", dk, kshape), ("dv", dv, kshape)):
        if t is None:
            t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        else:
            _check(t, name, torch.bfloat16, shape, dev)
        outs.append(t)
    nbytes = bwd_workspace_bytes(B, H, N, d) if d in (64, 128) else 0
    if workspace is None:
        workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
    bm_ptr, mb = _mask_args(blockmask, N, mask_block, dev, Nk)
    ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_ptr(dev))
    grads = (outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr())
    if Nk != N:
        rc = load_library().fa_bwd_nqk(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       do.data_ptr(), lse.data_ptr(), B, H, N, Nk, d, scale,
                                       int(bool(causal)), bm_ptr, mb, *grads, *ws)
        if rc != FA_OK:
            raise LibfaError(rc, "fa_bwd_nqk")
        return tuple(outs)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
            lse.data_ptr(), B, H, N, d, scale, int(bool(causal)), bm_ptr, mb)
    if dropout_p:
        rc = load_library().fa_bwd_dropout(*ptrs, float(dropout_p), int(seed), int(offset),
                                           *grads, *ws)
        if rc != FA_OK:
            raise LibfaError(rc, "fa_bwd_dropout")
        return tuple(outs)
    rc = load_library().fa_bwd(*ptrs, *grads, *ws)
    if rc != FA_OK:
        raise LibfaError(rc, "fa_bwd")
    return tuple(outs)


def backward_noalloc(q, k, v, o, do, lse, scale: float | None = None, causal: bool = False,
                     blockmask=None, mask_block: int = 128, dq=None, dk=None, dv=None):
    """fa_bwd_noalloc: the gradients of fa_bwd with D kept in the library's static
    scratch instead of a workspace (B*H*N <= NOALLOC_MAX_ROWS).  Pass dq, dk, dv to
    allocate nothing here either."""
    torch = _torch()
    _check(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _check(t, name, torch.bfloat16, q.shape, dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    scale = default_scale(d) if scale is None else float(scale)
    outs = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        else:
            _check(t, name, torch.bfloat16, q.shape, dev)
        outs.append(t)
    bm_ptr, mb = _mask_args(blockmask, N, mask_block, dev)
    rc = load_library().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       do.data_ptr(), lse.data_ptr(), B, H, N, d, scale,
                                       int(bool(causal)), bm_ptr, mb, outs[0].data_ptr(),
                                       outs[1].data_ptr(), outs[2].data_ptr(), _stream_ptr(dev))
    if rc != FA_OK:
        raise LibfaError(rc, "fa_bwd_noalloc")
    return tuple(outs)


def dropout_keep_mask(B: int, H: int, N: int, dropout_p: float, seed: int = 0, offset: int = 0,
                      device="cuda"):
    """The dropout stream's keep decisions as a uint8 [B, H, N, N] tensor (1 = kept)."""
    torch = _torch()
    keep = torch.empty((B, H, N, N), dtype=torch.uint8, device=device)
    rc = load_library().fa_dropout_keep_mask(B, H, N, float(dropout_p), int(seed), int(offset),
                                             keep.data_ptr(), _stream_ptr(keep.device))
    if rc != FA_OK:
        raise LibfaError(rc, "fa_dropout_keep_mask")
    return keep


def bwd_dsum(o, do, dsum=None):
    """Stage 1 of the backward: D = rowsum(dO * O) as float32 [B, H, N]."""
    torch = _torch()
    _check(o, "o", torch.bfloat16)
    B, H, N, d = o.shape
    _check(do, "do", torch.bfloat16, o.shape, o.device)
    if dsum is None:
        dsum = torch.empty((B, H, N), dtype=torch.float32, device=o.device)
    else:
        _check(dsum, "dsum", torch.float32, (B, H, N), o.device)
    rc = load_library().fa_bwd_dsum(o.data_ptr(), do.data_ptr(), B, H, N, d, dsum.data_ptr(),
                                    _stream_ptr(o.device))
    if rc != FA_OK:
        raise LibfaError(rc, "fa_bwd_dsum")
    return dsum


def _stage_inputs(q, k, v, do, lse, dsum):
    torch = _torch()
    _check(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    for name, t in (("k", k), ("v", v), ("do", do)):
        _check(t, name, torch.bfloat16, q.shape, q.device)
    B, H, N, d = q.shape
    _check(lse, "lse", torch.float32, (B, H, N), q.device)
    _check(dsum, "dsum", torch.float32, (B, H, N), q.device)
    return B, H, N, d


def bwd_dkdv(q, k, v, do, lse, dsum, scale=None, causal=False, blockmask=None, mask_block=128,
             dk=None, dv=None):
    """Stage 2 of the backward: dK, dV (needs D from bwd_dsum)."""
    torch = _torch()
    B, H, N, d = _stage_inputs(q, k, v, do, lse, dsum)
    scale = default_scale(d) if scale is None else float(scale)
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check(dk, "dk", torch.bfloat16, q.shape, q.device)
    _check(dv, "dv", torch.bfloat16, q.shape, q.device)
    bm_ptr, mb = _mask_args(blockmask, N, mask_block, q.device)
    rc = load_library().fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), dsum.data_ptr(), B, H, N, d, scale,
                                    int(bool(causal)), bm_ptr, mb, dk.data_ptr(), dv.data_ptr(),
                                    _stream_ptr(q.device))
    if rc != FA_OK:
        raise LibfaError(rc, "fa_bwd_dkdv")
    return dk, dv


def bwd_dq(q, k, v, do, lse, dsum, scale=None, causal=False, blockmask=None, mask_block=128,
           dq=None):
    """Stage 3 of the backward: dQ (needs D from bwd_dsum)."""
    torch = _torch()
    B, H, N, d = _stage_inputs(q, k, v, do, lse, dsum)
    scale = default_scale(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    _check(dq, "dq", torch.bfloat16, q.shape, q.device)
    bm_ptr, mb = _mask_args(blockmask, N, mask_block, q.device)
    rc = load_library().fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), dsum.data_ptr(), B, H, N, d, scale,
                                  int(bool(causal)), bm_ptr, mb, dq.data_ptr(),
                                  _stream_ptr(q.device))
    if rc != FA_OK:
        raise LibfaError(rc, "fa_bwd_dq")
    return dq


def bwd_dq_dsum(q, k, v, o, do, lse, scale=None, causal=False, blockmask=None, mask_block=128,
                dsum=None, dq=None):
    """dQ and D in one launch (the first half of backward); returns (dq, dsum)."""
    torch = _torch()
    _check(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _check(t, name, torch.bfloat16, q.shape, q.device)
    B, H, N, d = q.shape
    _check(lse, "lse", torch.float32, (B, H, N), q.device)
    if dsum is None:
        dsum = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(dsum, "dsum", torch.float32, (B, H, N), q.device)
    scale = default_scale(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    _check(dq, "dq", torch.bfloat16, q.shape, q.device)
    bm_ptr, mb = _mask_args(blockmask, N, mask_block, q.device)
    rc = load_library().fa_bwd_dq_dsum(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       do.data_ptr(), lse.data_ptr(), B, H, N, d, scale,
                                       int(bool(causal)), bm_ptr, mb, dsum.data_ptr(),
                                       dq.data_ptr(), _stream_ptr(q.device))
    if rc != FA_OK:
        raise LibfaError(rc, "fa_bwd_dq_dsum")
    return dq, dsum


class FlashAttention:
    """torch.autograd.Function adapter over forward/backward (built lazily)."""

    _fn = None

    @classmethod
    def apply(cls, q, k, v, scale=None, causal=False, blockmask=None, mask_block=128):
        if cls._fn is None:
            torch = _torch()

            class _Fn(torch.autograd.Function):
                @staticmethod
                def forward(ctx, q, k, v, scale, causal, blockmask, mask_block):
                    o, lse = forward(q, k, v, scale, causal, blockmask, mask_block)
                    ctx.save_for_backward(q, k, v, o, lse)
                    ctx.args = (scale, causal, blockmask, mask_block)
                    return o

                @staticmethod
                def backward(ctx, do):
                    q, k, v, o, lse = ctx.saved_tensors
                    dq, dk, dv = backward(q, k, v, o, do.contiguous(), lse, *ctx.args)
                    return dq, dk, dv, None, None, None, None

            cls._fn = _Fn
        return cls._fn.apply(q, k, v, scale, causal, blockmask, mask_block)


def splitkv_num_splits(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    """The split count fa_fwd_splitkv chooses by itself."""
    return int(load_library().fa_fwd_splitkv_num_splits(B, H, Nq, Nk, d))


def forward_splitkv(q, k, v, scale: float | None = None, causal: bool = False, blockmask=None,
                    mask_block: int = 128, num_splits: int = 0, out=None, lse=None):
    """Forward with the key axis split across workgroups (decoding shapes: few
    query rows, long K/V).  Same results as ``forward`` up to rounding."""
    torch = _torch()
    _check(q, "q", torch.bfloat16)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    dev = q.device
    _check(k, "k", torch.bfloat16, (B, H, Nk, d), dev)
    _check(v, "v", torch.bfloat16, (B, H, Nk, d), dev)
    scale = default_scale(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, q.shape, dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    lib = load_library()
    nbytes = int(lib.fa_fwd_splitkv_workspace_bytes(B, H, N, Nk, d, int(num_splits)))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    bm_ptr, mb = _mask_args(blockmask, N, mask_block, dev, Nk)
    rc = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, Nk, d, scale,
                            int(bool(causal)), bm_ptr, mb, int(num_splits), ws.data_ptr(),
                            ws.numel(), out.data_ptr(), lse.data_ptr(), _stream_ptr(dev))
    if rc != FA_OK:
        raise LibfaError(rc, "fa_fwd_splitkv")
    return out, lse



def forward_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float,
                scale: float | None = None, causal: bool = False, blockmask=None,
                mask_block: int = 128, out=None, lse=None):
    """FP8 forward (fa_fwd_fp8).  q, k, v: [B, H, N, 128] E4M3 codes, as
    torch.float8_e4m3fn or torch.uint8 tensors; element x stands for
    value(x) * descale of its tensor.  Returns (o bf16, lse fp32)."""
    torch = _torch()
    codes = (torch.float8_e4m3fn, torch.uint8)
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B, H, N, d] tensor")
    if q.dtype not in codes:
        raise TypeError(f"q must be float8_e4m3fn or uint8 codes, got {q.dtype}")
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype, (B, H, N, d), dev)
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    else:
        _check(out, "out", torch.bfloat16, (B, H, N, d), dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    else:
        _check(lse, "lse", torch.float32, (B, H, N), dev)
    bm_ptr, mb = _mask_args(blockmask, N, mask_block, dev)
    rc = load_library().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d, scale,
                                   float(q_descale), float(k_descale), float(v_descale),
                                   int(bool(causal)), bm_ptr, mb, out.data_ptr(),
                                   lse.data_ptr(), _stream_ptr(dev))
    if rc != FA_OK:
        raise LibfaError(rc, "fa_fwd_fp8")
    return out, lse
