"""ORACLE — test infrastructure only.

Plain CPU fp64 softmax attention (``attn_oracle.c``) behind a thin ctypes
wrapper.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package; the GPU library never does, and the
two share no code.  Inputs are numpy arrays: float64, float32, or uint16
holding bf16 bit patterns; the C side widens each element exactly to fp64.
FP8 (OCP E4M3) inputs are decoded to fp64 here (``e4m3_decode``) and scaled
by their per-tensor descales before the same attention.

Every function follows the plain definition of bidirectional multi-head
softmax attention (NVIDIA Technical Blog "Scaling AI Inference Across
Multiple GPUs Using NVIDIA TensorRT with Multi-Device Inference Support",
sections "Context parallelism", "AllGather KV", "Ring Attention",
"DeepSpeed Ulysses"); see the header of ``attn_oracle.c`` for the formula.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_KINDS = {np.dtype(np.float64): 0, np.dtype(np.float32): 1, np.dtype(np.uint16): 2}


_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile liboracle.so with gcc (IEEE fp64, no fast-math), OpenMP over query rows; with
    sanitize, liboracle_san.so instead (clang, AddressSanitizer + UndefinedBehaviorSanitizer, the
    same source and flags otherwise), for the sanitizer test."""
    out = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        if sanitize:
            import synth
            cmd = ["/opt/rocm/llvm/bin/clang"] + synth.SANITIZE_FLAGS + [
                "-fopenmp", "-fPIC", "-shared", "-std=c11", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        else:
            cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("ORACLE_LIBRARY") or _LIB  # another build of the same source
            if path == _LIB and not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(path)
            i64, vp, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
            lib.oracle_attention.argtypes = [i64] * 5 + [dbl, vp, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int,
                                                        i64, i64, vp, vp, vp, ctypes.c_int]
            lib.oracle_attention.restype = ctypes.c_int
            lib.oracle_lse_merge.argtypes = [i64, i64, i64, vp, vp, vp, vp]
            lib.oracle_lse_merge.restype = ctypes.c_int
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
        return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _arr(x: np.ndarray) -> Tuple[np.ndarray, int]:
    x = np.ascontiguousarray(x)
    if x.dtype not in _KINDS:
        raise TypeError("oracle inputs must be float64, float32 or uint16 (bf16 bits), got %s" % x.dtype)
    return x, _KINDS[x.dtype]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              kv_range: Optional[Tuple[int, int]] = None, q_rows: Optional[Sequence[int]] = None,
              want_p: bool = False, nthreads: int = 0):
    """Softmax attention in fp64.

    q: [B, H, Sq, D]; k, v: [B, H, Skv, D].  ``q_rows`` selects query rows
    (the result then has len(q_rows) rows); ``kv_range`` = (lo, hi) restricts
    the keys.  Returns (O [B,H,R,D] fp64, LSE [B,H,R] fp64[, P [B,H,R,n]]).
    """
    if q_rows is not None:
        q = q[:, :, np.asarray(q_rows, dtype=np.int64), :]
    q, qk = _arr(q)
    k, kk = _arr(k)
    v, vk = _arr(v)
    B, H, R, D = q.shape
    Skv = k.shape[2]
    assert k.shape == (B, H, Skv, D) and v.shape == (B, H, Skv, D), (q.shape, k.shape, v.shape)
    lo, hi = kv_range if kv_range is not None else (0, Skv)
    o = np.empty((B, H, R, D), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    p = np.empty((B, H, R, hi - lo), dtype=np.float64) if want_p else None
    rc = _load().oracle_attention(B, H, R, Skv, D, float(scale), q.ctypes.data, qk, k.ctypes.data, kk,
                                  v.ctypes.data, vk, lo, hi, o.ctypes.data, lse.ctypes.data,
                                  None if p is None else p.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments (rc=%d)" % rc)
    return (o, lse, p) if want_p else (o, lse)


def lse_merge(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """Merge results over disjoint key ranges (any shapes [..., D] / [...]), in fp64."""
    n = len(o_parts)
    assert n == len(lse_parts) and n >= 1
    shape = o_parts[0].shape
    D = shape[-1]
    rows = int(np.prod(shape[:-1]))
    os_ = [np.ascontiguousarray(x, dtype=np.float64) for x in o_parts]
    ls_ = [np.ascontiguousarray(x, dtype=np.float64) for x in lse_parts]
    for a, b in zip(os_, ls_):
        assert a.shape == shape and b.shape == shape[:-1]
    optr = (ctypes.c_void_p * n)(*[a.ctypes.data for a in os_])
    lptr = (ctypes.c_void_p * n)(*[b.ctypes.data for b in ls_])
    o = np.empty(shape, dtype=np.float64)
    lse = np.empty(shape[:-1], dtype=np.float64)
    rc = _load().oracle_lse_merge(n, rows, D, optr, lptr, o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_lse_merge rejected its arguments (rc=%d)" % rc)
    return o, lse


def chunk_partials(q, k, v, scale, chunk_lens: Sequence[int], q_rows=None, nthreads: int = 0
                   ) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Per-chunk (O_c, LSE_c) over consecutive key ranges of the given lengths."""
    out, off = [], 0
    for n in chunk_lens:
        out.append(attention(q, k, v, scale, kv_range=(off, off + n), q_rows=q_rows, nthreads=nthreads))
        off += n
    assert off == k.shape[2]
    return out


# ---- DeepSpeed-Ulysses re-layout (blog section "DeepSpeed Ulysses": each rank trades its
# sequence slice of all heads for the whole sequence of one head group).  Pure data movement;
# the definitions below are index maps, exact for any dtype.

def ulysses_pack(x: np.ndarray, n: int) -> np.ndarray:
    """x [B, H, S, D] -> packed [n, S, B, H/n, D] with packed[j, s, b, h', d] = x[b, j*H/n + h', s, d]."""
    B, H, S, D = x.shape
    assert H % n == 0
    Hg = H // n
    out = np.empty((n, S, B, Hg, D), dtype=x.dtype)
    for j in range(n):
        for b in range(B):
            # head group j of batch b, [Hg, S, D] -> [S, Hg, D]
            out[j, :, b] = np.transpose(x[b, j * Hg:(j + 1) * Hg], (1, 0, 2))
    return out


def ulysses_unpack(packed: np.ndarray) -> np.ndarray:
    """packed [n, S, B, Hg, D] -> x [B, n*Hg, S, D], the inverse of ulysses_pack."""
    n, S, B, Hg, D = packed.shape
    x = np.empty((B, n * Hg, S, D), dtype=packed.dtype)
    for j in range(n):
        for b in range(B):
            x[b, j * Hg:(j + 1) * Hg] = np.transpose(packed[j, :, b], (1, 0, 2))
    return x


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64, exactly.

    Sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.  Exponent
    field 0: (-1)^s * m * 2^-9 (zero and subnormals); otherwise
    (-1)^s * (1 + m/8) * 2^(e-7).  Codes 0x7F and 0xFF are NaN; the format has
    no infinities.  Straight from the format definition, element by element.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def attention_e4m3(q, k, v, q_descale: float, k_descale: float, v_descale: float, scale: float,
                   q_rows=None, nthreads: int = 0):
    """Attention of E4M3-coded tensors: the plain definition applied to the decoded
    values times their per-tensor descales (each product exact in fp64)."""
    if q_rows is not None:
        q = q[:, :, np.asarray(q_rows, dtype=np.int64), :]
    qd = e4m3_decode(q) * float(q_descale)
    kd = e4m3_decode(k) * float(k_descale)
    vd = e4m3_decode(v) * float(v_descale)
    return attention(qd, kd, vd, scale, nthreads=nthreads)
