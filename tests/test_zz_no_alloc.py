"""attn_shard_fwd_noalloc against attn_shard_fwd (fused schedule, caller's workspace).

The allocation-free entry point keeps the balanced tail's partials in the library's static
scratch array instead of a workspace; with the same plan it must give the same result, bit for
bit.  Two calls in a row, the second smaller (the array keeps the first call's contents), then a
shape without a tail and the fp32 path; each through the C ABI, against the workspace entry point
and, on sampled rows, against the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import assert_parity, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_sequence_dit_amd import attn
    attn.load()


def A():
    from long_sequence_dit_amd import attn
    return attn


def _case(B, H, Sq, lens, order, D=128, seed=40, kind=synth.KIND_BF16, out_dtype=torch.bfloat16):
    Skv = sum(lens)
    q = synth.normal_rows(seed, 0, B, H, Sq, D, kind=kind)
    k = synth.normal_rows(seed, 1, B, H, Skv, D, kind=kind)
    v = synth.normal_rows(seed, 2, B, H, Skv, D, kind=kind)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    ws = torch.empty(max(A().shard_workspace_size(B, H, Sq, D, len(lens), "fused"), 1), dtype=torch.uint8,
                     device="cuda")
    o_ws, l_ws = A().shard_fwd(qd, kd, vd, lens, order, mode="fused", workspace=ws, out_dtype=out_dtype)
    out = torch.empty((B, H, Sq, D), dtype=out_dtype, device="cuda")
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    o_na, l_na = A().shard_fwd_noalloc(qd, kd, vd, lens, order, out, lse)
    torch.cuda.synchronize()
    assert o_na.data_ptr() == out.data_ptr() and l_na.data_ptr() == lse.data_ptr()
    assert torch.equal(o_na, o_ws), float((o_na.float() - o_ws.float()).abs().max())
    assert torch.equal(l_na, l_ws), float((l_na - l_ws).abs().max())
    rows = sorted({0, 1, Sq // 2, Sq - 1})
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(D), q_rows=rows)
    assert_parity(o_na[:, :, rows], l_na[:, :, rows], o_ref, l_ref, fp32=kind == synth.KIND_F32,
                  what="noalloc B%d H%d Sq%d lens %s" % (B, H, Sq, lens))
    return ws.numel()


def test_noalloc_matches_workspace_entry_point_twice():
    # 3 query tiles against 141 key tiles: the tail runs as 256 runs of about 1.7 key tiles
    need1 = _case(1, 3, 600, (3000, 6000), (1, 0))
    assert need1 > 1
    # then a smaller call: 2 query tiles against 79 key tiles (fewer slots than the first call)
    need2 = _case(1, 2, 300, (5000,), None, seed=41)
    assert need2 > 1


def test_noalloc_without_tail_and_fp32():
    # 256 query tiles fill one round: no tail, so the scratch array is not touched
    assert _case(1, 16, 4096, (700, 300), (1, 0), seed=42) == 1
    # fp32 path (no tail in the fp32 kernel), D = 64
    _case(1, 2, 256, (64, 64, 64, 64), None, D=64, seed=43, kind=synth.KIND_F32, out_dtype=torch.float32)


def test_noalloc_argument_errors_touch_nothing():
    q = torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, 1, 8, 96), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 1, 8), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(A().AttnError):
        A().shard_fwd_noalloc(q, q, q, (8,), None, out, lse)  # D = 96: unsupported
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
