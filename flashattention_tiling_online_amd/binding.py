"""Thin ctypes binding of libfa.so (include/fa.h): argument marshalling only.

Every step of the attention forward runs in the library's gfx950 kernels; torch
is used for device memory and the current HIP stream.  If the library has not
been built the first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")
DEBUG_LIB_PATH = os.path.join(PKG, "libfa_debug.so")  # the full-barrier check build

FA_DTYPE_F32, FA_DTYPE_F16, FA_DTYPE_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH, FA_ERR_SCRATCH = 0, 1, 2, 3, 4
FA_STATIC_SCRATCH_BYTES = 64 << 20  # include/fa.h

# symbols include/fa.h declares
EXPORTS = ("fa_fwd", "fa_fwd_masked", "fa_fwd_split", "fa_fwd_split_workspace",
           "fa_fwd_split_static", "fa_merge", "fa_split_hint", "fa_bwd", "fa_bwd_masked",
           "fa_bwd_workspace", "fa_fwd_dropout", "fa_bwd_dropout", "fa_status_str",
           "fa_tile_rows")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"libfa call failed: {fa_status_str(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the library (libfa.so, or the check build libfa_debug.so) and
    declare the argument and result types of every entry point."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m flashattention_tiling_online_amd.build --all)")
    L = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    L.fa_fwd.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_void_p, i64, i64, i64, i64, i64,
                                                  ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                                  ctypes.c_void_p]
    L.fa_fwd.restype = ctypes.c_int
    L.fa_status_str.argtypes = [ctypes.c_int]
    L.fa_status_str.restype = ctypes.c_char_p
    L.fa_tile_rows.argtypes = [ctypes.c_int, i64, ctypes.c_int]
    L.fa_tile_rows.restype = ctypes.c_int
    L.fa_fwd_split.argtypes = L.fa_fwd.argtypes[:-1] + [ctypes.c_int, ctypes.c_void_p, i64,
                                                        ctypes.c_void_p]
    L.fa_fwd_split.restype = ctypes.c_int
    L.fa_fwd_masked.argtypes = [ctypes.c_void_p] * 4 + [i64, i64] + [ctypes.c_void_p] * 2 + [
        i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    L.fa_fwd_masked.restype = ctypes.c_int
    L.fa_fwd_split_static.argtypes = L.fa_fwd.argtypes[:-1] + [ctypes.c_int, ctypes.c_void_p]
    L.fa_fwd_split_static.restype = ctypes.c_int
    L.fa_fwd_split_workspace.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    L.fa_fwd_split_workspace.restype = i64
    L.fa_merge.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, i64, i64, i64, i64,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.fa_merge.restype = ctypes.c_int
    L.fa_split_hint.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    L.fa_split_hint.restype = ctypes.c_int
    L.fa_bwd.argtypes = [ctypes.c_void_p] * 9 + [i64, i64, i64, i64, i64, ctypes.c_int,
                                                  ctypes.c_float, ctypes.c_int,
                                                  ctypes.c_void_p, i64, ctypes.c_void_p]
    L.fa_bwd.restype = ctypes.c_int
    L.fa_bwd_masked.argtypes = [ctypes.c_void_p] * 4 + [i64, i64] + [ctypes.c_void_p] * 6 + [
        i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
        i64, ctypes.c_void_p]
    L.fa_bwd_masked.restype = ctypes.c_int
    L.fa_bwd_workspace.argtypes = [i64, i64, i64, i64]
    L.fa_bwd_workspace.restype = i64
    drop = [ctypes.c_float, ctypes.c_uint64]
    L.fa_fwd_dropout.argtypes = L.fa_fwd.argtypes[:12] + drop + L.fa_fwd.argtypes[12:]
    L.fa_fwd_dropout.restype = ctypes.c_int
    L.fa_bwd_dropout.argtypes = L.fa_bwd.argtypes[:16] + drop + L.fa_bwd.argtypes[16:]
    L.fa_bwd_dropout.restype = ctypes.c_int
    return L


def fa_status_str(status: int) -> str:
    return lib().fa_status_str(int(status)).decode()


def fa_tile_rows(dtype: int, d: int, causal: bool) -> int:
    return lib().fa_tile_rows(int(dtype), int(d), int(bool(causal)))


def fa_fwd_raw(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int, Nk: int,
               d: int, causal: int, scale: float, dtype: int, stream: int) -> int:
    """Direct call with integer device pointers; returns the fa_status_t code."""
    return lib().fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, int(causal), float(scale),
                        int(dtype), stream)


def fa_fwd_masked_raw(q: int, k: int, v: int, mask: int, mask_b: int, mask_h: int, o: int,
                      lse: int, B: int, H: int, Nq: int, Nk: int, d: int, causal: int,
                      scale: float, dtype: int, stream: int) -> int:
    """Direct call of fa_fwd_masked with integer device pointers; returns the status code."""
    return lib().fa_fwd_masked(q, k, v, mask, int(mask_b), int(mask_h), o, lse, B, H, Nq, Nk, d,
                               int(causal), float(scale), int(dtype), stream)


def fa_fwd_split_raw(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int, Nk: int,
                     d: int, causal: int, scale: float, dtype: int, n_splits: int,
                     workspace: int, workspace_bytes: int, stream: int) -> int:
    """Direct call of fa_fwd_split with integer device pointers; returns the status code."""
    return lib().fa_fwd_split(q, k, v, o, lse, B, H, Nq, Nk, d, int(causal), float(scale),
                              int(dtype), int(n_splits), workspace, int(workspace_bytes), stream)


def fa_fwd_split_static_raw(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int,
                            Nk: int, d: int, causal: int, scale: float, dtype: int, n_splits: int,
                            stream: int) -> int:
    """Direct call of fa_fwd_split_static (no workspace, nothing allocated); returns the
    status code."""
    return lib().fa_fwd_split_static(q, k, v, o, lse, B, H, Nq, Nk, d, int(causal), float(scale),
                                     int(dtype), int(n_splits), stream)


def fa_merge_raw(o_parts: int, lse_parts: int, n_parts: int, B: int, H: int, Nq: int, d: int,
                 o: int, lse: int, dtype: int, stream: int) -> int:
    """Direct call of fa_merge with integer device pointers; returns the status code."""
    return lib().fa_merge(o_parts, lse_parts, int(n_parts), B, H, Nq, d, o, lse, int(dtype),
                          stream)


def fa_bwd_raw(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int,
               B: int, H: int, Nq: int, Nk: int, d: int, causal: int, scale: float, dtype: int,
               workspace: int, workspace_bytes: int, stream: int) -> int:
    """Direct call of fa_bwd with integer device pointers; returns the status code."""
    return lib().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, int(causal),
                        float(scale), int(dtype), workspace, int(workspace_bytes), stream)


def fa_bwd_masked_raw(q: int, k: int, v: int, mask: int, mask_b: int, mask_h: int, o: int,
                      lse: int, dout: int, dq: int, dk: int, dv: int, B: int, H: int, Nq: int,
                      Nk: int, d: int, causal: int, scale: float, dtype: int, workspace: int,
                      workspace_bytes: int, stream: int) -> int:
    """Direct call of fa_bwd_masked with integer device pointers; returns the status code."""
    return lib().fa_bwd_masked(q, k, v, mask, int(mask_b), int(mask_h), o, lse, dout, dq, dk, dv,
                               B, H, Nq, Nk, d, int(causal), float(scale), int(dtype), workspace,
                               int(workspace_bytes), stream)


def fa_fwd_dropout_raw(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int,
                       Nk: int, d: int, causal: bool, scale: float, p_drop: float, seed: int,
                       dtype: int, stream: int) -> int:
    """Direct call of fa_fwd_dropout with integer device pointers; returns the status code."""
    return lib().fa_fwd_dropout(q, k, v, o, lse, B, H, Nq, Nk, d, int(causal), float(scale),
                                float(p_drop), int(seed) & 0xFFFFFFFFFFFFFFFF, int(dtype), stream)


def fa_bwd_dropout_raw(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int,
                       dv: int, B: int, H: int, Nq: int, Nk: int, d: int, causal: bool,
                       scale: float, p_drop: float, seed: int, dtype: int, workspace: int,
                       workspace_bytes: int, stream: int) -> int:
    """Direct call of fa_bwd_dropout with integer device pointers; returns the status code."""
    return lib().fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, int(causal),
                                float(scale), float(p_drop), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                int(dtype), workspace, workspace_bytes, stream)


def fa_bwd_workspace(B: int, H: int, Nq: int, d: int) -> int:
    return lib().fa_bwd_workspace(B, H, Nq, d)


def fa_fwd_split_workspace(B: int, H: int, Nq: int, d: int, n_splits: int) -> int:
    return lib().fa_fwd_split_workspace(B, H, Nq, d, int(n_splits))


def fa_split_hint(B: int, H: int, Nq: int, Nk: int, d: int, causal: bool, dtype: int) -> int:
    return lib().fa_split_hint(B, H, Nq, Nk, d, int(bool(causal)), int(dtype))


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_DTYPE_F32, torch.float16: FA_DTYPE_F16,
             torch.bfloat16: FA_DTYPE_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor [B,H,N,d]")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same GPU")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != (B, H, Nk, d):
        raise ValueError("k and v must be [B,H,Nk,d] with q's B, H and d")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    return B, H, Nq, Nk, d


def _check_buf(name, t, shape, dtype, device):
    """A caller-supplied buffer: a contiguous tensor of `shape` and `dtype` on `device`
    (the library sees only its address, so a wrong one would send the kernels out of
    bounds or to host memory)."""
    if not hasattr(t, "is_cuda") or not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _check_workspace(t, need, device):
    """A caller-supplied workspace: a contiguous GPU buffer of at least `need` bytes."""
    if not hasattr(t, "is_cuda") or not t.is_cuda or t.device != device:
        raise ValueError(f"workspace must be a GPU tensor on {device}")
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if t.numel() * t.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    return t


def _outputs_fwd(q, B, H, Nq, o, lse):
    """o [B,H,Nq,d] in q's dtype and lse [B,H,Nq] fp32: checked if given, else allocated
    (on the current stream, which the caller has made the launch stream)."""
    import torch
    if o is None:
        o = torch.empty_like(q)
    else:
        _check_buf("o", o, q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        _check_buf("lse", lse, (B, H, Nq), torch.float32, q.device)
    return o, lse


def _launch_stream(stream, device):
    """The stream to enqueue on (default: torch's current stream on `device`)."""
    import torch
    return torch.cuda.current_stream(device) if stream is None else stream


def fa_fwd_split(q, k, v, causal: bool = False, scale: float | None = None, n_splits=None,
                 o=None, lse=None, workspace=None, stream=None):
    """fa_fwd computed over key ranges and merged (fa_fwd_split).

    n_splits defaults to fa_split_hint(...).  The fp32 workspace for the partial
    states is allocated with torch when not given (a uint8 GPU tensor of at least
    fa_fwd_split_workspace(...) bytes may be passed instead).  Buffers the binding
    allocates are allocated on the launch stream, so that torch does not hand their
    memory to other work before the kernels on that stream are done with it.
    """
    import torch
    B, H, Nq, Nk, d = _check_qkv(q, k, v)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if n_splits is None:
        n_splits = max(1, fa_split_hint(B, H, Nq, Nk, d, causal, code))
    stream = _launch_stream(stream, q.device)
    need = fa_fwd_split_workspace(B, H, Nq, d, n_splits)
    with torch.cuda.stream(stream):
        o, lse = _outputs_fwd(q, B, H, Nq, o, lse)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        else:
            _check_workspace(workspace, max(need, 0), q.device)
    st = fa_fwd_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          B, H, Nq, Nk, d, int(bool(causal)), scale, code, n_splits,
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          stream.cuda_stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse


def fa_merge(o_parts, lse_parts, dtype=None, o=None, lse=None, stream=None):
    """Fold partial states o_parts [P,B,H,Nq,d], lse_parts [P,B,H,Nq] (fp32 GPU tensors)
    into (o [B,H,Nq,d] of ``dtype``, lse [B,H,Nq] fp32) with fa_merge."""
    import torch
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("o_parts and lse_parts must be float32")
    if not (o_parts.is_cuda and lse_parts.is_cuda and o_parts.is_contiguous()
            and lse_parts.is_contiguous() and o_parts.dim() == 5
            and lse_parts.shape == o_parts.shape[:4] and lse_parts.device == o_parts.device):
        raise ValueError("o_parts must be [P,B,H,Nq,d] and lse_parts [P,B,H,Nq], contiguous, "
                         "on one GPU")
    P, B, H, Nq, d = o_parts.shape
    dev = o_parts.device
    if dtype is None:
        dtype = o.dtype if o is not None else torch.bfloat16
    stream = _launch_stream(stream, dev)
    with torch.cuda.stream(stream):
        if o is None:
            o = torch.empty((B, H, Nq, d), dtype=dtype, device=dev)
        else:
            _check_buf("o", o, (B, H, Nq, d), dtype, dev)
        if lse is None:
            lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
        else:
            _check_buf("lse", lse, (B, H, Nq), torch.float32, dev)
    st = fa_merge_raw(o_parts.data_ptr(), lse_parts.data_ptr(), P, B, H, Nq, d, o.data_ptr(),
                      lse.data_ptr(), _dtype_code(o), stream.cuda_stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse


def _bwd_buffers(q, k, v, o, lse, dout, dq, dk, dv, workspace, stream):
    """Checks and allocations shared by fa_bwd and fa_bwd_dropout."""
    import torch
    B, H, Nq, Nk, d = _check_qkv(q, k, v)
    dev = q.device
    _check_buf("o", o, q.shape, q.dtype, dev)
    _check_buf("dout", dout, q.shape, q.dtype, dev)
    _check_buf("lse", lse, (B, H, Nq), torch.float32, dev)
    stream = _launch_stream(stream, dev)
    need = fa_bwd_workspace(B, H, Nq, d)
    with torch.cuda.stream(stream):
        dq = torch.empty_like(q) if dq is None else _check_buf("dq", dq, q.shape, q.dtype, dev)
        dk = torch.empty_like(k) if dk is None else _check_buf("dk", dk, k.shape, k.dtype, dev)
        dv = torch.empty_like(v) if dv is None else _check_buf("dv", dv, v.shape, v.dtype, dev)
        if workspace is None:
            workspace = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
        else:
            _check_workspace(workspace, max(need, 0), dev)
    return (B, H, Nq, Nk, d), dq, dk, dv, workspace, stream


def fa_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, dq=None,
           dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV of the attention forward (fa_bwd) from the forward's o and lse and the
    output gradient dout; the fp32 workspace for D = rowsum(dO o O) is allocated with
    torch (on the launch stream) when not given."""
    (B, H, Nq, Nk, d), dq, dk, dv, workspace, stream = _bwd_buffers(
        q, k, v, o, lse, dout, dq, dk, dv, workspace, stream)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = fa_bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Nq, Nk, d,
                    int(bool(causal)), scale, code, workspace.data_ptr(),
                    workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != FA_OK:
        raise FAError(st)
    return dq, dk, dv


def fa_bwd_masked(q, k, v, mask, o, lse, dout, causal: bool = False, scale: float | None = None,
                  dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV of fa_fwd_masked's forward (fa_bwd_masked), with the same mask."""
    (B, H, Nq, Nk, d), dq, dk, dv, workspace, stream = _bwd_buffers(
        q, k, v, o, lse, dout, dq, dk, dv, workspace, stream)
    mb, mh = _check_mask(mask, B, H, Nq, Nk, q.device)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = fa_bwd_masked_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), mask.data_ptr(), mb, mh,
                           o.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                           dk.data_ptr(), dv.data_ptr(), B, H, Nq, Nk, d, int(bool(causal)),
                           scale, code, workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != FA_OK:
        raise FAError(st)
    return dq, dk, dv


def fa_fwd(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None,
           stream=None):
    """O, L = attention forward of torch tensors q [B,H,Nq,d], k, v [B,H,Nk,d] on the GPU.

    o and lse are allocated (torch, on the launch stream) when not given.  The kernel
    is enqueued on ``stream`` (default: torch's current stream) and the call returns
    at once.
    """
    import torch
    B, H, Nq, Nk, d = _check_qkv(q, k, v)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):
        o, lse = _outputs_fwd(q, B, H, Nq, o, lse)
    st = fa_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                    Nq, Nk, d, int(bool(causal)), scale, code, stream.cuda_stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse


def _check_mask(mask, B, H, Nq, Nk, device):
    """A caller mask: a contiguous int32 or uint32 GPU tensor [mask_b, mask_h, Nq,
    ceil(Nk/32)] with mask_b in {1, B} and mask_h in {1, H}."""
    import torch
    if not hasattr(mask, "is_cuda") or not mask.is_cuda or mask.device != device:
        raise ValueError(f"mask must be a GPU tensor on {device}")
    if mask.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise TypeError("mask must hold 32-bit words (int32 or uint32)")
    if not mask.is_contiguous() or mask.dim() != 4:
        raise ValueError("mask must be a contiguous 4-D tensor [mask_b, mask_h, Nq, W]")
    mb, mh, nq, w = mask.shape
    if mb not in (1, B) or mh not in (1, H) or nq != Nq or w != -(-Nk // 32):
        raise ValueError(f"mask must be [1 or {B}, 1 or {H}, {Nq}, {-(-Nk // 32)}], got "
                         f"{tuple(mask.shape)}")
    return mb, mh


def fa_fwd_masked(q, k, v, mask, causal: bool = False, scale: float | None = None, o=None,
                  lse=None, stream=None):
    """fa_fwd with a caller mask (fa_fwd_masked): ``mask`` holds the bit-packed rows
    [mask_b, mask_h, Nq, ceil(Nk/32)] (key k in bit k % 32 of word k // 32, set =
    visible).  A row with no visible key gets O = 0 and L = -inf."""
    import torch
    B, H, Nq, Nk, d = _check_qkv(q, k, v)
    mb, mh = _check_mask(mask, B, H, Nq, Nk, q.device)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):
        o, lse = _outputs_fwd(q, B, H, Nq, o, lse)
    st = fa_fwd_masked_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), mask.data_ptr(), mb, mh,
                           o.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d, int(bool(causal)),
                           scale, code, stream.cuda_stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse


def fa_fwd_dropout(q, k, v, p_drop: float, seed: int, causal: bool = False,
                   scale: float | None = None, o=None, lse=None, stream=None):
    """fa_fwd with dropout on P (fa_fwd_dropout): O = (P o Z) V, L as without dropout."""
    import torch
    B, H, Nq, Nk, d = _check_qkv(q, k, v)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):
        o, lse = _outputs_fwd(q, B, H, Nq, o, lse)
    st = fa_fwd_dropout_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr(), B, H, Nq, Nk, d, bool(causal), scale, p_drop, seed,
                            code, stream.cuda_stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse


def fa_bwd_dropout(q, k, v, o, lse, dout, p_drop: float, seed: int, causal: bool = False,
                   scale: float | None = None, dq=None, dk=None, dv=None, workspace=None,
                   stream=None):
    """fa_bwd with the dropout of fa_fwd_dropout (same p_drop and seed)."""
    (B, H, Nq, Nk, d), dq, dk, dv, workspace, stream = _bwd_buffers(
        q, k, v, o, lse, dout, dq, dk, dv, workspace, stream)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = fa_bwd_dropout_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(), B, H, Nq, Nk, d, bool(causal), scale, p_drop, seed,
                            code, workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != FA_OK:
        raise FAError(st)
    return dq, dk, dv
