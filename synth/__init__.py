"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This package holds no attention arithmetic: it draws N(0, 1) values from a
counter-based generator (Philox4x32-10 + Box-Muller, in ``synth_gen.c``),
scales them in fp64 and rounds them to fp32 or bf16.  Both sides of every
parity check read the same host buffers made here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

KIND_F64, KIND_F32, KIND_BF16 = 0, 1, 2

# Tensor ids of the counter-based streams.
TID_Q, TID_K, TID_V, TID_OUTLIER = 0, 1, 2, 3


_LIB_SAN = os.path.join(_HERE, "libsynth_san.so")
# clang of the ROCm toolchain, whose AddressSanitizer runtime the sanitized HIP library uses too
_CLANG = "/opt/rocm/llvm/bin/clang"
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-shared-libsan",
                  "-Wl,-rpath,/opt/rocm/llvm/lib"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile libsynth.so next to its source (plain gcc, OpenMP); with sanitize, libsynth_san.so
    instead (clang, AddressSanitizer + UndefinedBehaviorSanitizer), for the sanitizer test."""
    out = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        if sanitize:
            cmd = [_CLANG] + SANITIZE_FLAGS + ["-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        else:
            cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("SYNTH_LIBRARY") or _LIB  # another build of the same source
            if path == _LIB and not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(path)
            lib.synth_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
            lib.synth_philox4x32_10.restype = None
            lib.synth_raw_u32.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_void_p]
            lib.synth_raw_u32.restype = None
            lib.synth_normal_rows.argtypes = [ctypes.c_uint64, ctypes.c_uint32] + [ctypes.c_int64] * 6 + [
                ctypes.c_double, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
            lib.synth_normal_rows.restype = ctypes.c_int
            lib.synth_f32_to_bf16.argtypes = [ctypes.c_float]
            lib.synth_f32_to_bf16.restype = ctypes.c_uint16
            _lib = lib
        return _lib


def philox4x32_10(ctr, key):
    """One Philox4x32-10 block: 4 counter words and 2 key words in, 4 words out."""
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    lib.synth_philox4x32_10(c, k)
    return [int(x) for x in c]


def raw_u32(seed: int, tensor_id: int, first: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    _load().synth_raw_u32(seed, tensor_id, first, n, out.ctypes.data)
    return out


def normal_rows(seed, tensor_id, B, H, S, D, row_lo=0, row_hi=None, factor=1.0, row_factor=None,
                kind=KIND_BF16, out=None) -> np.ndarray:
    """Rows [row_lo, row_hi) of a [B, H, S, D] N(0,1)*factor tensor.

    bf16 results are returned as uint16 bit patterns.
    """
    if row_hi is None:
        row_hi = S
    dt = {KIND_F64: np.float64, KIND_F32: np.float32, KIND_BF16: np.uint16}[kind]
    shape = (B, H, row_hi - row_lo, D)
    if out is None:
        out = np.empty(shape, dtype=dt)
    assert out.shape == shape and out.dtype == dt and out.flags.c_contiguous
    rf = None
    if row_factor is not None:
        rf = np.ascontiguousarray(row_factor, dtype=np.float64)
        assert rf.shape == (S,)
    rc = _load().synth_normal_rows(seed, tensor_id, B, H, S, D, row_lo, row_hi, float(factor),
                                   None if rf is None else rf.ctypes.data, kind, out.ctypes.data)
    if rc != 0:
        raise ValueError("synth_normal_rows rejected its arguments (rc=%d)" % rc)
    return out


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    u16 = np.ascontiguousarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 by round-to-nearest-even, as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


E4M3_MAX = 448.0
_BLOCK = 1 << 20


def f64_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Values -> OCP FP8 E4M3 codes (uint8) by round-to-nearest-even.

    E4M3 (the "fn" variant): sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent field 0 holds subnormals m * 2^-9; no infinities, and codes
    0x7F / 0xFF are NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
    Every finite input must round to a magnitude <= 448 (scale inputs into
    range first); anything else raises.

    Within binade [2^e, 2^(e+1)), e >= -6, representable magnitudes are the
    multiples of 2^(e-3); below 2^-6 the step stays 2^-9.  With e clamped to
    >= -6 and q = round-half-even(|x| / 2^(e-3)), the code is 8 (e + 6) + q
    (a q of 16 carries into the next binade by the same formula).
    """
    x = np.asarray(x)
    if x.size > _BLOCK:  # elementwise: encode in blocks (large temporaries are slow to allocate)
        flat = x.reshape(-1)
        out = np.empty(flat.shape, dtype=np.uint8)
        for i in range(0, flat.size, _BLOCK):
            out[i:i + _BLOCK] = f64_to_e4m3_bits(flat[i:i + _BLOCK])
        return out.reshape(x.shape)
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("E4M3 encoding of a non-finite value")
    a = np.abs(x)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    q = np.rint(np.ldexp(a, (3 - e).astype(np.int32))).astype(np.int64)  # exact scaling, RNE
    code = 8 * (e + 6) + q
    code = np.where(a == 0.0, 0, code)
    if np.any(code > 0x7E):
        raise ValueError("E4M3 encoding: magnitude beyond 448 after rounding")
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def e4m3_quantize(x: np.ndarray):
    """Per-tensor E4M3 quantization: (codes, descale) with x ~= decode(codes) * descale.

    descale = max|x| / 448 in fp32, so the largest magnitude maps to 448; each element is
    divided by it in fp64 and rounded once.
    """
    x = np.asarray(x)
    amax = float(max(np.max(x), -np.min(x))) if x.size else 0.0
    descale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i in range(0, flat.size, _BLOCK):
        out[i:i + _BLOCK] = f64_to_e4m3_bits(flat[i:i + _BLOCK].astype(np.float64) / descale)
    return out.reshape(x.shape), descale


def outlier_rows(seed: int, S: int, count: int) -> np.ndarray:
    """`count` distinct row positions in [0, S), drawn without replacement.

    Position p gets the key (word p of stream TID_OUTLIER, p); the `count`
    smallest keys are chosen and returned sorted.
    """
    w = raw_u32(seed, TID_OUTLIER, 0, S).astype(np.uint64)
    keys = (w << np.uint64(32)) | np.arange(S, dtype=np.uint64)
    return np.sort(np.argsort(keys, kind="stable")[:count])
