"""GPU checks of the Ulysses re-layout (pack / unpack around the all-to-all) and of the one-GPU
Ulysses path: pack Q, K, V of the whole sequence, attend each head group on its packed view,
unpack the outputs.  Re-layout is exact: compared bit for bit with the oracle's index maps."""
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


def _bits(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("kind", ["bf16", "fp32"])
@pytest.mark.parametrize("B,H,S,D,n", [(1, 32, 333, 128, 8), (2, 6, 50, 64, 3), (3, 4, 17, 128, 1), (1, 4, 1, 64, 4)])
def test_pack_unpack_exact(kind, B, H, S, D, n):
    k = synth.KIND_BF16 if kind == "bf16" else synth.KIND_F32
    x = synth.normal_rows(7, 0, B, H, S, D, kind=k)
    xd = to_device(x)
    p = A().ulysses_pack(xd, n)
    torch.cuda.synchronize()
    want = oracle.ulysses_pack(x, n)
    got = _bits(p)
    assert np.array_equal(got.view(want.dtype) if kind == "bf16" else got, want)
    y = A().ulysses_unpack(p)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16) if kind == "bf16" else y, xd.view(torch.int16) if kind == "bf16" else xd)


def test_pack_from_and_unpack_into_bshd_views():
    B, H, S, D, n = 2, 8, 40, 128, 4
    x = synth.normal_rows(8, 0, B, H, S, D, kind=synth.KIND_BF16)
    xd = to_device(x)
    bshd = xd.permute(0, 2, 1, 3).contiguous()          # [B, S, H, D] storage
    view = bshd.permute(0, 2, 1, 3)                      # seen as [B, H, S, D]
    p = A().ulysses_pack(view, n)
    assert torch.equal(p, A().ulysses_pack(xd, n))
    out = torch.empty_like(bshd)
    A().ulysses_unpack(p, out=out.permute(0, 2, 1, 3))
    torch.cuda.synchronize()
    assert torch.equal(out, bshd)


def test_one_gpu_ulysses_path_matches_oracle():
    """Pack Q, K, V (all heads, whole sequence) into n head groups, run attention on each
    group's packed view, unpack: equals attention over all heads."""
    B, H, S, D, n = 1, 8, 700, 128, 4
    q, k, v = (synth.normal_rows(9, t, B, H, S, D, kind=synth.KIND_BF16) for t in range(3))
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(D))
    qp, kp, vp = (A().ulysses_pack(to_device(x), n) for x in (q, k, v))
    op = torch.empty_like(qp)
    lse = torch.empty((n, B, H // n, S), dtype=torch.float32, device="cuda")
    for j in range(n):
        gv = A().head_group_view
        A().shard_fwd(gv(qp, j), gv(kp, j), gv(vp, j), (S,), out=gv(op, j), lse=lse[j])
    o = A().ulysses_unpack(op)
    torch.cuda.synchronize()
    l = lse.permute(1, 0, 2, 3).reshape(B, H, S)
    assert_parity(o, l, o_ref, l_ref, what="one-GPU Ulysses path")
