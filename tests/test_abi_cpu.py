"""The C-ABI library on the host: it loads, exports what include/attn.h declares,
and rejects bad arguments with the documented status before any HIP call.

No call here reaches a kernel launch: every argument set is invalid, and the
library checks arguments before touching the HIP runtime.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def attn():
    from long_sequence_dit_amd import attn as a
    if not os.path.exists(a.lib_path()):
        import long_sequence_dit_amd.build as b
        b.build()
    a.load()
    return a


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src))


def test_exports_every_declared_symbol(attn):
    names = _declared()
    assert names == set(attn.EXPORTS)
    lib = ctypes.CDLL(attn.lib_path())
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(attn):
    lib = attn.load()
    assert lib.attn_abi_version() == 1
    for code in range(8):
        assert len(lib.attn_status_str(code)) > 0
    assert lib.attn_status_str(99) == b"unknown status"


def _st(b, h, s):
    from long_sequence_dit_amd.attn import Strides
    return Strides(b, h, s)


P = 0x10000  # an aligned, never dereferenced address


def _chunk(lib, q=P, k=P, v=P, o=P, lse=P, in_dt=BF16, o_dt=BF16, B=1, H=2, Sq=10, Skv=20, D=128, scale=0.1,
           qs=None, ks=None, vs=None, os_=None):
    c = _st(2 * 1000 * 128, 1000 * 128, 128)
    return lib.attn_chunk_fwd(q, qs or c, k, ks or c, v, vs or c, in_dt, B, H, Sq, Skv, D, scale, o, os_ or c, o_dt,
                              lse, None)


def test_chunk_fwd_argument_errors(attn):
    lib = attn.load()
    assert _chunk(lib, q=None) == NULL
    assert _chunk(lib, lse=None) == NULL
    assert _chunk(lib, k=None) == NULL
    assert _chunk(lib, in_dt=7) == DTYPE
    assert _chunk(lib, in_dt=F32, o_dt=BF16) == DTYPE
    assert _chunk(lib, D=96) == UNSUP
    assert _chunk(lib, D=256) == UNSUP
    assert _chunk(lib, Sq=-1) == SHAPE
    assert _chunk(lib, Skv=-1) == SHAPE
    assert _chunk(lib, scale=0.0) == SHAPE
    assert _chunk(lib, scale=float("nan")) == SHAPE
    assert _chunk(lib, scale=float("inf")) == SHAPE
    assert _chunk(lib, q=P + 2) == ALIGN
    assert _chunk(lib, lse=P + 4) == ALIGN
    assert _chunk(lib, qs=_st(0, 0, 129)) == ALIGN
    assert _chunk(lib, os_=_st(0, 3, 128)) == ALIGN
    assert _chunk(lib, ks=_st(-128, 0, 128)) == ALIGN
    # fp32 strides need a multiple of 4 elements, bf16 a multiple of 8
    assert _chunk(lib, in_dt=BF16, qs=_st(0, 0, 132)) == ALIGN
    # one head's K/V rows must span < 2 GiB on the bf16 path (32-bit buffer offsets)
    assert _chunk(lib, ks=_st(0, 0, 2**27)) == UNSUP
    assert _chunk(lib, vs=_st(0, 0, 2**24), Skv=2**7) == UNSUP
    # the limit covers the loads of the three tiles the kernel fetches past the last one
    assert _chunk(lib, ks=_st(0, 0, 2**22), Skv=128) == UNSUP  # (128 + 256) * 2^23 >= 2^31
    # empty problems are no-ops, even with NULL pointers
    assert _chunk(lib, q=None, k=None, v=None, o=None, lse=None, Sq=0) == OK
    assert _chunk(lib, q=None, k=None, v=None, o=None, lse=None, B=0) == OK


def test_lse_merge_argument_errors(attn):
    lib = attn.load()
    arr = (ctypes.c_void_p * 2)(P, P)
    c = _st(2 * 10 * 128, 10 * 128, 128)
    m = lambda n=2, op=arr, lp=arr, D=128, o=P, lse=P, odt=BF16, os_=c, Sq=10: lib.attn_lse_merge(
        n, op, lp, 1, 2, Sq, D, o, os_, odt, lse, None)
    assert m(n=0) == SHAPE
    assert m(n=65) == UNSUP
    assert m(D=32) == UNSUP
    assert m(odt=5) == DTYPE
    assert m(op=None) == NULL
    assert m(o=None) == NULL
    assert m(op=(ctypes.c_void_p * 2)(P, None)) == NULL
    assert m(lp=(ctypes.c_void_p * 2)(P, P + 8)) == ALIGN
    assert m(o=P + 2) == ALIGN
    assert m(Sq=0, op=None, lp=None, o=None, lse=None) == OK


def _shard(lib, lens=(10, 10), order=None, flags=4, ws=P, ws_bytes=1 << 30, D=128, q=P, in_dt=BF16, o_dt=BF16,
           Sq=10):
    c = _st(2 * 1000 * 128, 1000 * 128, 128)
    n = len(lens)
    la = (ctypes.c_int32 * max(n, 1))(*lens)
    oa = None if order is None else (ctypes.c_int32 * len(order))(*order)
    return lib.attn_shard_fwd(q, c, P, c, P, c, in_dt, 1, 2, Sq, D, 0.1, n, la, oa, flags, ws, ws_bytes, P, c, o_dt,
                              P, None)


def _al(n):
    return -(-n // 256) * 256


def _tail_room(n_slots, D=128):
    """Partial slots of the balanced tail: 256 rows of D fp32 values, then 256 fp32 LSEs, each."""
    return _al(n_slots * 256 * D * 4) + _al(n_slots * 256 * 4)


WQ = 16 * 64 * 4  # the work queues of a persistent launch: 16 counters, 256 bytes apart


def test_shard_fwd_argument_errors(attn):
    lib = attn.load()
    assert _shard(lib, lens=()) == SHAPE
    assert _shard(lib, lens=(1,) * 65) == UNSUP
    assert _shard(lib, lens=(10, -1)) == SHAPE
    assert _shard(lib, lens=(2**30, 2**30)) == SHAPE
    assert _shard(lib, order=(0, 0)) == SHAPE
    assert _shard(lib, order=(0, 2)) == SHAPE
    assert _shard(lib, order=(1, -1)) == SHAPE
    assert _shard(lib, flags=0) == UNSUP
    assert _shard(lib, flags=3) == UNSUP
    tail = _tail_room(256 + 2)  # room for the balanced tail: one run per CU, 2 query tiles
    for flags, n_slots in ((1, 2), (2, 1)):  # n-way and online keep fp32 partials in the workspace
        assert _shard(lib, ws=None, flags=flags) == WS
        need = lib.attn_shard_workspace_size(1, 2, 10, 128, 2, flags)
        slots = need - tail  # the chunk slots are required, the tail's room is optional
        assert slots == n_slots * (-(-20 * 128 * 4 // 256) * 256 + -(-20 * 4 // 256) * 256)
        assert _shard(lib, ws_bytes=slots - 1, flags=flags) == WS
        assert _shard(lib, ws=P + 8, ws_bytes=need, flags=flags) == ALIGN
    assert _shard(lib, D=80) == UNSUP
    assert _shard(lib, q=None) == NULL
    assert _shard(lib, in_dt=F32, o_dt=BF16) == DTYPE
    assert _shard(lib, q=None, Sq=0) == OK


def test_workspace_sizes(attn):
    lib = attn.load()
    rows = 1 * 16 * 5520
    slot = -(-rows * 128 * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    # fused: no chunk partials.  A shape of more than one round of query tiles (256 rows each;
    # the CPU build assumes 256 CUs) gets the work queues of a persistent launch; one whose tiles
    # leave the last round part-full (16 heads x 22 tiles = 352: 96 in the last round) also room
    # for the balanced tail: a slot of 256 rows x (D + 1) fp32 per run (up to 4 runs per CU) and
    # per tail tile, whatever the chunking; a shape filling whole rounds (16 x 16 tiles) none.
    # n-way keeps every chunk's fp32 partial and online one running result, followed by the same
    # room (each chunk's launch may use it).
    tail = WQ + _tail_room(4 * 256 + 96)
    assert lib.attn_shard_workspace_size(1, 16, 5520, 128, 8, 1) == 8 * slot + tail   # n-way
    assert lib.attn_shard_workspace_size(1, 16, 5520, 128, 8, 2) == 1 * slot + tail   # online
    assert lib.attn_shard_workspace_size(1, 16, 5520, 128, 8, 4) == tail
    assert lib.attn_shard_workspace_size(1, 16, 5520, 128, 1, 4) == tail  # one chunk: same kernel
    # 2768 tiles: 208 in the last round
    assert lib.attn_shard_workspace_size(1, 16, 44160, 128, 8, 4) == WQ + _tail_room(4 * 256 + 208)
    assert lib.attn_shard_workspace_size(1, 16, 4096, 128, 8, 4) == 0
    assert lib.attn_shard_workspace_size(1, 32, 4096, 128, 8, 4) == WQ  # two full rounds: queues only
    assert lib.attn_shard_workspace_size(1, 3, 4096, 128, 8, 4) == _tail_room(256 + 48)  # one round
    assert lib.attn_shard_workspace_size(1, 16, 5520, 64, 8, 4) == WQ + _tail_room(4 * 256 + 96, 64)
    assert lib.attn_shard_workspace_size(1, 16, 5520, 96, 8, 4) == 0
    assert lib.attn_shard_workspace_size(1, 16, 5520, 128, 8, 3) == 0


def test_ulysses_relayout_argument_errors(attn):
    lib = attn.load()
    c = _st(4 * 8 * 128, 8 * 128, 128)
    pack = lambda **kw: lib.attn_ulysses_pack(kw.get("x", P), kw.get("xs", c), kw.get("dt", BF16), kw.get("B", 1),
                                              kw.get("H", 8), kw.get("S", 4), kw.get("D", 128), kw.get("n", 4),
                                              kw.get("out", P), None)
    unpack = lambda **kw: lib.attn_ulysses_unpack(kw.get("inp", P), kw.get("dt", BF16), 1, kw.get("H", 8), 4, 128,
                                                  kw.get("n", 4), kw.get("x", P), kw.get("xs", c), None)
    assert pack(dt=9) == DTYPE
    assert pack(D=96) == UNSUP
    assert pack(n=3) == SHAPE and pack(n=0) == SHAPE and pack(H=-8) == SHAPE
    assert pack(x=None) == NULL and pack(out=None) == NULL
    assert pack(x=P + 8) == ALIGN and pack(xs=_st(0, 0, 4)) == ALIGN
    assert pack(x=None, out=None, S=0) == OK and pack(x=None, out=None, B=0) == OK
    assert unpack(dt=9) == DTYPE and unpack(n=3) == SHAPE
    assert unpack(inp=None) == NULL and unpack(x=P + 8) == ALIGN


def test_fp8_argument_errors(attn):
    lib = attn.load()
    c = _st(2 * 1000 * 128, 1000 * 128, 128)
    need = lib.attn_fp8_workspace_size(1, 2, 10, 20, 128)
    assert need == 1 * 2 * 1 * 8192          # V^T tiles of 64 keys; no tail for 2 query tiles of 1 key tile
    assert lib.attn_fp8_workspace_size(1, 2, 10, 65, 128) == 2 * 2 * 8192
    assert lib.attn_fp8_workspace_size(1, 2, 10, 20, 64) == 0 and lib.attn_fp8_workspace_size(1, 2, 10, 0, 128) == 0
    # 16 heads x 173 query tiles against 690 key tiles leave 208 tiles in the last round of 256 CUs
    # (the CPU build assumes 256): room for the balanced tail after V^T; 16 x 16 tiles fill it
    vt = 16 * 690 * 8192
    # a persistent launch (2768 tiles x 690 key tiles): the work queues, then a slot per run: each
    # of the 208 tail tiles cut into 3 parts (parts of at least 192 FP8 key tiles)
    assert lib.attn_fp8_workspace_size(1, 16, 44160, 44160, 128) == vt + WQ + _tail_room(3 * 208)
    assert lib.attn_fp8_workspace_size(1, 16, 4096, 44160, 128) == vt

    def f(q=P, k=P, v=P, o=P, lse=P, ws=P, ws_bytes=need, B=1, H=2, Sq=10, Skv=20, D=128, scale=0.1, dq=1.0, dk=1.0,
          dv=1.0, odt=BF16, qs=None, ks=None, vs=None, os_=None):
        return lib.attn_chunk_fwd_fp8(q, qs or c, k, ks or c, v, vs or c, dq, dk, dv, B, H, Sq, Skv, D, scale, ws,
                                      ws_bytes, o, os_ or c, odt, lse, None)

    assert f(odt=7) == DTYPE
    assert f(D=64) == UNSUP
    assert f(Sq=-1) == SHAPE and f(Skv=-2) == SHAPE
    assert f(scale=0.0) == SHAPE and f(dq=float("nan")) == SHAPE and f(dv=-1.0) == SHAPE and f(dk=float("inf")) == SHAPE
    assert f(q=None) == NULL and f(k=None) == NULL and f(ws=None) == NULL
    assert f(q=P + 8) == ALIGN and f(ws=P + 8) == ALIGN
    assert f(qs=_st(0, 0, 136)) == ALIGN      # E4M3 strides: multiples of 16 bytes
    assert f(os_=_st(0, 0, 132)) == ALIGN     # bf16 output: multiples of 8 elements
    assert f(ws_bytes=need - 1) == WS
    assert f(ks=_st(0, 0, 2 ** 24)) == UNSUP  # one head's K rows must span < 2 GiB
    # ... including the four tiles fetched past the end: (200 + 320) * 2^22 >= 2^31 > (200 + 256) * 2^22
    assert f(ks=_st(0, 0, 2 ** 22), Skv=200) == UNSUP
    assert f(Skv=2 ** 23, ws_bytes=1 << 62) == UNSUP
    # no-ops, even with NULL pointers
    assert f(q=None, k=None, v=None, o=None, lse=None, ws=None, Sq=0) == OK
    assert f(q=None, k=None, v=None, o=None, lse=None, ws=None, H=0) == OK


def test_bench_tail_rule_matches_the_library(attn):
    """bench.py reports which kernels a step launches with its own copies of the balanced tail's
    and the persistent launch's rules; the FP8 workspace size (V^T tiles, plus the work queues
    exactly when the launch is persistent, plus the tail's slots exactly when the tail runs)
    shows the library's decisions, which must agree for every shape (256 CUs on the CPU build)."""
    import bench
    lib = attn.load()
    for B, H, Sq, Skv in [(1, 16, 44160, 44160), (1, 4, 44160, 44160), (1, 16, 5520, 44160), (1, 24, 4608, 4608),
                          (1, 16, 4096, 44160), (1, 3, 200, 5000), (1, 3, 200, 3000), (1, 2, 10, 20),
                          (2, 7, 1000, 9000), (1, 1, 300, 8323072), (1, 32, 4096, 44160), (1, 40, 4096, 3000)]:
        vt = B * H * -(-Skv // 64) * 8192
        n_q, T = B * H * -(-Sq // 256), -(-Skv // 64)
        extra = lib.attn_fp8_workspace_size(B, H, Sq, Skv, 128) - vt - (WQ if bench.persistent_launch(n_q, T, 256, 2) else 0)
        assert extra >= 0 and extra % 256 == 0, (B, H, Sq, Skv)
        assert (extra > 0) == bench.tail_runs(n_q, T, 256), (B, H, Sq, Skv)
