"""The largest key counts the entry points accept, checked through a closed form.

Attention over a key block repeated r times equals attention over the block: every key's weight
is shared by its r copies, so O is unchanged and LSE grows by ln r.  A 65,536-key block repeated
127 times gives 8,323,072 keys, whose bf16 K and V rows (2.13 GB each) sit just under the 2^31-byte
limit of the 32-bit buffer offsets, and whose E4M3 rows sit under the FP8 entry's 2^23-key limit.
The repetition is made on the device, so the oracle runs on the block alone.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu

BLOCK, REPS, SQ, D = 65536, 127, 300, 128
SKV = BLOCK * REPS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_sequence_dit_amd import attn
    attn.load()


def A():
    from long_sequence_dit_amd import attn
    return attn


def test_sizes_are_at_the_limits():
    assert (SKV + 256) * D * 2 < 2 ** 31 <= (SKV + 256 + 65536) * D * 2   # bf16 guard of the API
    assert SKV < 2 ** 23 and (SKV + 320) * D < 2 ** 31                   # fp8 guards


def test_bf16_repeated_block_at_max_keys():
    q = synth.normal_rows(41, 0, 1, 1, SQ, D)
    k = synth.normal_rows(41, 1, 1, 1, BLOCK, D)
    v = synth.normal_rows(41, 2, 1, 1, BLOCK, D)
    scale = 1 / math.sqrt(D)
    o_ref, l_ref = oracle.attention(q, k, v, scale)
    l_ref = l_ref + math.log(REPS)
    qd = to_device(q)
    kd, vd = to_device(k).repeat(1, 1, REPS, 1), to_device(v).repeat(1, 1, REPS, 1)
    assert kd.shape[2] == SKV
    # fused shard: the balanced tail spreads 2 query tiles x 130,048 key tiles over the CUs
    o, l = A().shard_fwd(qd, kd, vd, (SKV,), None, mode="fused")
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, what="bf16 %d keys, fused shard" % SKV)
    # single chunk, no workspace: one workgroup per query tile walks all 130,048 tiles
    o2, l2 = A().chunk_fwd(qd, kd, vd, scale)
    torch.cuda.synchronize()
    assert_parity(o2, l2, o_ref, l_ref, what="bf16 %d keys, one chunk" % SKV)


def test_fp8_repeated_block_at_max_keys():
    src = {"q": synth.normal_rows(43, 0, 1, 1, SQ, D, kind=synth.KIND_F32),
           "k": synth.normal_rows(43, 1, 1, 1, BLOCK, D, kind=synth.KIND_F32),
           "v": synth.normal_rows(43, 2, 1, 1, BLOCK, D, kind=synth.KIND_F32)}
    codes, ds = {}, {}
    for n, x in src.items():
        codes[n], ds[n] = synth.e4m3_quantize(x)
    qd, kd, vd = (oracle.e4m3_decode(codes[n]) * ds[n] for n in ("q", "k", "v"))
    scale = 1 / math.sqrt(D)
    o_ref, l_ref, P = oracle.attention(qd, kd, vd, scale, want_p=True)
    a_abs, _ = oracle.attention(qd, kd, np.abs(vd), scale)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    kg, vg = dev(codes["k"]).repeat(1, 1, REPS, 1), dev(codes["v"]).repeat(1, 1, REPS, 1)
    o, l = A().chunk_fwd_fp8(dev(codes["q"]), kg, vg, ds["q"], ds["k"], ds["v"], scale)
    torch.cuda.synchronize()
    o, l = to_f64(o), to_f64(l)
    # the FP8 bound of tests/test_gpu_fp8.py, on the block: each key's probability is shared by
    # its copies, so the relative and the small-probability terms are those of the block
    pmax = P.max(axis=-1, keepdims=True)
    small = P < 2.0 ** -11 * pmax
    s_small = np.einsum("bhrj,bhjd->bhrd", small.astype(np.float64), np.abs(vd))
    bound = 2.0 ** -4 * a_abs + 2.0 ** -15 * pmax * s_small + 2.0 ** -8 * np.abs(o_ref) + 1e-6
    err = np.abs(o - o_ref)
    lerr = np.abs(l - (l_ref + math.log(REPS)))
    print("fp8 %d keys: O max err %.3g (worst err/bound %.3f), LSE max err %.3g"
          % (SKV, err.max(), float((err / bound).max()), lerr.max()), flush=True)
    assert np.all(np.isfinite(o)) and np.all(err <= bound)
    assert np.all(lerr <= math.log1p(2.0 ** -4) + 2.0 ** -15 * pmax[..., 0] * small.sum(-1) + 1e-5)
