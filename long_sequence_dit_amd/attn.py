"""ctypes binding of libattn.so — argument marshalling only.

Each function checks that its torch tensors are device tensors of a supported
dtype with a unit stride on the last dimension, allocates any output the
caller did not pass (torch provides device memory and streams), and hands
raw pointers, element strides and the current HIP stream to the C entry point
of the same name.  Every step of the computation runs in the library's HIP
kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Sequence

import torch

# LSDIT_ATTN_LIBRARY selects another build of the same sources (the sanitizer test loads the
# AddressSanitizer build of the host code this way).
_LIB_PATH = os.environ.get("LSDIT_ATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                                 "libattn.so")
_lock = threading.Lock()
_lib = None

ATTN_F32, ATTN_BF16 = 0, 1
MERGE_NWAY, MERGE_ONLINE, MERGE_FUSED = 1, 2, 4
_MODES = {"nway": MERGE_NWAY, "online": MERGE_ONLINE, "fused": MERGE_FUSED}
MAX_CHUNKS = 64

STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_DTYPE", 4: "ATTN_ERR_ALIGN",
          5: "ATTN_ERR_UNSUPPORTED", 6: "ATTN_ERR_WORKSPACE", 7: "ATTN_ERR_HIP"}

# Every symbol include/attn.h declares.
EXPORTS = ("attn_chunk_fwd", "attn_lse_merge", "attn_shard_workspace_size", "attn_shard_fwd",
           "attn_shard_fwd_noalloc", "attn_ulysses_pack", "attn_ulysses_unpack", "attn_fp8_workspace_size", "attn_chunk_fwd_fp8",
           "attn_status_str", "attn_abi_version")


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("s", ctypes.c_int64)]


class AttnError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s failed: %s (%s)" % (what, STATUS.get(code, code), _status_str(code)))


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libattn.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libattn.so is not built (expected at %s); run __graft_entry__.build()" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, f32, sz, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint32
        lib.attn_chunk_fwd.argtypes = [vp, Strides, vp, Strides, vp, Strides, ctypes.c_int, i32, i32, i32, i32, i32,
                                       f32, vp, Strides, ctypes.c_int, vp, vp]
        lib.attn_chunk_fwd.restype = ctypes.c_int
        lib.attn_lse_merge.argtypes = [i32, vp, vp, i32, i32, i32, i32, vp, Strides, ctypes.c_int, vp, vp]
        lib.attn_lse_merge.restype = ctypes.c_int
        lib.attn_shard_workspace_size.argtypes = [i32, i32, i32, i32, i32, u32]
        lib.attn_shard_workspace_size.restype = sz
        lib.attn_shard_fwd.argtypes = [vp, Strides, vp, Strides, vp, Strides, ctypes.c_int, i32, i32, i32, i32, f32,
                                       i32, vp, vp, u32, vp, sz, vp, Strides, ctypes.c_int, vp, vp]
        lib.attn_shard_fwd.restype = ctypes.c_int
        lib.attn_shard_fwd_noalloc.argtypes = [vp, Strides, vp, Strides, vp, Strides, ctypes.c_int, i32, i32, i32,
                                               i32, f32, i32, vp, vp, vp, Strides, ctypes.c_int, vp, vp]
        lib.attn_shard_fwd_noalloc.restype = ctypes.c_int
        lib.attn_ulysses_pack.argtypes = [vp, Strides, ctypes.c_int, i32, i32, i32, i32, i32, vp, vp]
        lib.attn_ulysses_pack.restype = ctypes.c_int
        lib.attn_ulysses_unpack.argtypes = [vp, ctypes.c_int, i32, i32, i32, i32, i32, vp, Strides, vp]
        lib.attn_ulysses_unpack.restype = ctypes.c_int
        lib.attn_fp8_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        lib.attn_fp8_workspace_size.restype = sz
        lib.attn_chunk_fwd_fp8.argtypes = [vp, Strides, vp, Strides, vp, Strides, f32, f32, f32, i32, i32, i32, i32,
                                           i32, f32, vp, sz, vp, Strides, ctypes.c_int, vp, vp]
        lib.attn_chunk_fwd_fp8.restype = ctypes.c_int
        lib.attn_status_str.argtypes = [ctypes.c_int]
        lib.attn_status_str.restype = ctypes.c_char_p
        lib.attn_abi_version.argtypes = []
        lib.attn_abi_version.restype = i32
        _lib = lib
        return lib


def _status_str(code: int) -> str:
    try:
        return load().attn_status_str(code).decode()
    except Exception:  # library not loadable: only the code is known
        return "?"


def _check(code: int, what: str):
    if code != 0:
        raise AttnError(code, what)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t.dtype)


def _bhsd(t: torch.Tensor, name: str) -> Strides:
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dim() != 4:
        raise ValueError("%s must be [B, H, S, D], got shape %s" % (name, tuple(t.shape)))
    if t.stride(3) != 1 and t.shape[3] > 1:
        raise ValueError("%s must have a unit stride on D" % name)
    return Strides(*t.stride()[:3])


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _side_stream(stream):
    """The torch stream a call runs on when that is not the current stream (else None)."""
    if stream is None:
        return None
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    return None if s.cuda_stream == torch.cuda.current_stream().cuda_stream else s


def _used_on(stream, *tensors):
    """Tensors this binding allocated (on the current stream) for a call enqueued on another
    stream: tell the caching allocator that stream uses them, so that their memory is not handed
    to a later allocation before the call's kernels are done with it."""
    s = _side_stream(stream)
    if s is not None:
        for t in tensors:
            if t is not None:
                t.record_stream(s)


def _scale(scale, D):
    return float(1.0 / math.sqrt(D) if scale is None else scale)


def chunk_fwd(q, k, v, scale=None, out=None, lse=None, out_dtype=None, stream=None):
    """Attention of every query row against one chunk of keys -> (O, LSE)."""
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if tuple(k.shape) != (B, H, Skv, D) or tuple(v.shape) != (B, H, Skv, D):
        raise ValueError("k, v must be [B, H, Skv, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    out_dtype = out_dtype or q.dtype
    own = []
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=out_dtype, device=q.device)
        own.append(out)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
        own.append(lse)
    if not lse.is_contiguous() or lse.dtype != torch.float32:
        raise ValueError("lse must be contiguous fp32 [B, H, Sq]")
    _used_on(stream, *own)
    rc = load().attn_chunk_fwd(q.data_ptr(), _bhsd(q, "q"), k.data_ptr(), _bhsd(k, "k"), v.data_ptr(),
                               _bhsd(v, "v"), _dt(q), B, H, Sq, Skv, D, _scale(scale, D), out.data_ptr(),
                               _bhsd(out, "out"), _dt(out), lse.data_ptr(), _stream_ptr(stream))
    _check(rc, "attn_chunk_fwd")
    return out, lse


def fp8_workspace_size(B, H, Sq, Skv, D) -> int:
    return int(load().attn_fp8_workspace_size(B, H, Sq, Skv, D))


def _e4m3(t: torch.Tensor, name: str) -> torch.Tensor:
    """E4M3 codes as a uint8 view (torch.float8_e4m3fn tensors are accepted as they are)."""
    if t.dtype == torch.uint8:
        return t
    if t.dtype == getattr(torch, "float8_e4m3fn", None):
        return t.view(torch.uint8)
    raise TypeError("%s must hold E4M3 codes (uint8 or float8_e4m3fn), got %s" % (name, t.dtype))


def chunk_fwd_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float, scale=None, out=None, lse=None,
                  out_dtype=torch.bfloat16, workspace=None, stream=None):
    """FP8 (E4M3) attention of every query row against one chunk of keys -> (O, LSE)."""
    q, k, v = _e4m3(q, "q"), _e4m3(k, "k"), _e4m3(v, "v")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if tuple(k.shape) != (B, H, Skv, D) or tuple(v.shape) != (B, H, Skv, D):
        raise ValueError("k, v must be [B, H, Skv, D] matching q")
    own = []
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=out_dtype, device=q.device)
        own.append(out)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
        own.append(lse)
    if not lse.is_contiguous() or lse.dtype != torch.float32:
        raise ValueError("lse must be contiguous fp32 [B, H, Sq]")
    need = fp8_workspace_size(B, H, Sq, Skv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        own.append(workspace)
    _used_on(stream, *own)
    rc = load().attn_chunk_fwd_fp8(q.data_ptr(), _bhsd(q, "q"), k.data_ptr(), _bhsd(k, "k"), v.data_ptr(),
                                   _bhsd(v, "v"), float(q_descale), float(k_descale), float(v_descale), B, H, Sq,
                                   Skv, D, _scale(scale, D), workspace.data_ptr(), workspace.numel(),
                                   out.data_ptr(), _bhsd(out, "out"), _dt(out), lse.data_ptr(), _stream_ptr(stream))
    _check(rc, "attn_chunk_fwd_fp8")
    return out, lse


def lse_merge(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor], out=None, lse=None,
              out_dtype=torch.bfloat16, stream=None):
    """Merge fp32 results over disjoint key sets by their LSE -> (O, LSE)."""
    n = len(o_parts)
    if n != len(lse_parts) or n < 1:
        raise ValueError("need matching, non-empty lists of parts")
    B, H, Sq, D = o_parts[0].shape
    for o_, l_ in zip(o_parts, lse_parts):
        if tuple(o_.shape) != (B, H, Sq, D) or not o_.is_contiguous() or o_.dtype != torch.float32:
            raise ValueError("o parts must be contiguous fp32 [B, H, Sq, D]")
        if tuple(l_.shape) != (B, H, Sq) or not l_.is_contiguous() or l_.dtype != torch.float32:
            raise ValueError("lse parts must be contiguous fp32 [B, H, Sq]")
        if not o_.is_cuda or not l_.is_cuda:
            raise ValueError("parts must be GPU tensors")
    own = []
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=out_dtype, device=o_parts[0].device)
        own.append(out)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=o_parts[0].device)
        own.append(lse)
    _used_on(stream, *own)
    optr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in o_parts])
    lptr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in lse_parts])
    rc = load().attn_lse_merge(n, optr, lptr, B, H, Sq, D, out.data_ptr(), _bhsd(out, "out"), _dt(out),
                               lse.data_ptr(), _stream_ptr(stream))
    _check(rc, "attn_lse_merge")
    return out, lse


def shard_workspace_size(B, H, Sq, D, n_chunks, mode="fused") -> int:
    return int(load().attn_shard_workspace_size(B, H, Sq, D, n_chunks, _MODES[mode]))


def shard_fwd(q, k, v, chunk_lens: Sequence[int], order: Optional[Sequence[int]] = None, mode: str = "fused",
              scale=None, out=None, lse=None, workspace: Optional[torch.Tensor] = None, out_dtype=None,
              stream=None):
    """Query rows against the whole key sequence, chunk by chunk in `order` -> (O, LSE)."""
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if tuple(k.shape) != (B, H, Skv, D) or tuple(v.shape) != (B, H, Skv, D):
        raise ValueError("k, v must be [B, H, Skv, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    n = len(chunk_lens)
    lens = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in chunk_lens])
    ordp = None if order is None else (ctypes.c_int32 * max(len(order), 1))(*[int(x) for x in order])
    flags = _MODES[mode]
    need = shard_workspace_size(B, H, Sq, D, n, mode) if n >= 1 else 0
    own = []
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=out_dtype, device=q.device)
        own.append(out)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
        own.append(lse)
    _used_on(stream, *own)
    rc = load().attn_shard_fwd(q.data_ptr(), _bhsd(q, "q"), k.data_ptr(), _bhsd(k, "k"), v.data_ptr(),
                               _bhsd(v, "v"), _dt(q), B, H, Sq, D, _scale(scale, D), n, lens, ordp, flags, ws_ptr,
                               ws_bytes, out.data_ptr(), _bhsd(out, "out"), _dt(out), lse.data_ptr(),
                               _stream_ptr(stream))
    _check(rc, "attn_shard_fwd")
    return out, lse


def shard_fwd_noalloc(q, k, v, chunk_lens: Sequence[int], order: Optional[Sequence[int]], out, lse, scale=None,
                      stream=None):
    """shard_fwd with the fused schedule and no workspace: the library keeps the balanced tail's
    partials in its static scratch array.  Allocates nothing: the caller passes `out` and `lse`."""
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if tuple(k.shape) != (B, H, Skv, D) or tuple(v.shape) != (B, H, Skv, D):
        raise ValueError("k, v must be [B, H, Skv, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if tuple(out.shape) != (B, H, Sq, D):
        raise ValueError("out must be [B, H, Sq, D]")
    if tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous() or lse.dtype != torch.float32:
        raise ValueError("lse must be contiguous fp32 [B, H, Sq]")
    n = len(chunk_lens)
    lens = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in chunk_lens])
    ordp = None if order is None else (ctypes.c_int32 * max(len(order), 1))(*[int(x) for x in order])
    rc = load().attn_shard_fwd_noalloc(q.data_ptr(), _bhsd(q, "q"), k.data_ptr(), _bhsd(k, "k"), v.data_ptr(),
                                       _bhsd(v, "v"), _dt(q), B, H, Sq, D, _scale(scale, D), n, lens, ordp,
                                       out.data_ptr(), _bhsd(out, "out"), _dt(out), lse.data_ptr(),
                                       _stream_ptr(stream))
    _check(rc, "attn_shard_fwd_noalloc")
    return out, lse


def ulysses_pack(x, n: int, packed=None, stream=None):
    """Head groups of x [B, H, S, D] -> packed [n, S, B, H/n, D] (part j goes to rank j)."""
    B, H, S, D = x.shape
    if H % n:
        raise ValueError("H must be a multiple of n")
    if packed is None:
        packed = torch.empty((n, S, B, H // n, D), dtype=x.dtype, device=x.device)
        _used_on(stream, packed)
    if not packed.is_contiguous() or packed.dtype != x.dtype or tuple(packed.shape) != (n, S, B, H // n, D):
        raise ValueError("packed must be contiguous [n, S, B, H/n, D] of x's dtype")
    rc = load().attn_ulysses_pack(x.data_ptr(), _bhsd(x, "x"), _dt(x), B, H, S, D, n, packed.data_ptr(),
                                  _stream_ptr(stream))
    _check(rc, "attn_ulysses_pack")
    return packed


def ulysses_unpack(packed, out=None, stream=None):
    """packed [n, S, B, Hg, D] -> [B, n*Hg, S, D] (or into `out`, any [B, H, S, D] view)."""
    n, S, B, Hg, D = packed.shape
    if not packed.is_contiguous():
        raise ValueError("packed must be contiguous")
    if out is None:
        out = torch.empty((B, n * Hg, S, D), dtype=packed.dtype, device=packed.device)
        _used_on(stream, out)
    if tuple(out.shape) != (B, n * Hg, S, D) or out.dtype != packed.dtype:
        raise ValueError("out must be [B, n*Hg, S, D] of packed's dtype")
    rc = load().attn_ulysses_unpack(packed.data_ptr(), _dt(packed), B, n * Hg, S, D, n, out.data_ptr(),
                                    _bhsd(out, "out"), _stream_ptr(stream))
    _check(rc, "attn_ulysses_unpack")
    return out


def head_group_view(packed, j: int):
    """Part j of a packed buffer ([S, B, Hg, D]) as the [B, Hg, S, D] view attention takes."""
    return packed[j].permute(1, 2, 0, 3)
