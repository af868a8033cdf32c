"""The bf16 kernel's persistent dispatch: one workgroup per CU taking items (whole query tiles,
then the balanced tail's runs) from per-XCD work queues.

Which workgroup takes an item must not change any result: every item writes its own rows or
partial slots.  Launches of several rounds with enough work per CU run persistent by themselves;
the library's debug switches force it (LSDIT_DEBUG_PERSIST=1) or forbid it (=0) and fix the
tail (LSDIT_DEBUG_TAIL: "ranges" for one run of equal units per CU, as a launch of one workgroup
per item has; r for r parts per tail tile), so that these checks run at sizes the oracle
finishes in seconds: bitwise against the one-workgroup-per-item dispatch with the same tail,
bitwise repeatable, and with the tail tiles cut into parts against the oracle.
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


def _inputs(B, H, Sq, Skv, D, seed):
    return tuple(synth.normal_rows(seed, i, B, H, S, D, kind=synth.KIND_BF16)
                 for i, S in enumerate((Sq, Skv, Skv)))


def _run(qd, kd, vd, lens, order, mode, monkeypatch, persist, tail=None, out_dtype=torch.float32):
    monkeypatch.setenv("LSDIT_DEBUG_PERSIST", persist)
    if tail is None:
        monkeypatch.delenv("LSDIT_DEBUG_TAIL", raising=False)
    else:
        monkeypatch.setenv("LSDIT_DEBUG_TAIL", str(tail))
    o, l = A().shard_fwd(qd, kd, vd, lens, order, mode=mode, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, l


# 300 query tiles (20 heads x 15): 256 in the first round, 44 in the tail, against 79 key tiles;
# 768 tiles (48 heads x 16): three full rounds, no tail
SHAPES = [(1, 20, 3600, 5000), (1, 48, 4096, 1000)]


@pytest.mark.parametrize("mode", ["fused", "online", "nway"])
@pytest.mark.parametrize("shape", SHAPES)
def test_persistent_dispatch_matches_one_workgroup_per_item(shape, mode, monkeypatch):
    B, H, Sq, Skv = shape
    D = 128
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=41)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    lens, order = (Skv // 3, Skv - Skv // 3), (1, 0)
    print("persistent vs static: shape %s mode %s" % (shape, mode), flush=True)
    o_s, l_s = _run(qd, kd, vd, lens, order, mode, monkeypatch, "0")
    o_p, l_p = _run(qd, kd, vd, lens, order, mode, monkeypatch, "1", tail="ranges")
    assert torch.equal(o_s, o_p) and torch.equal(l_s, l_p)


@pytest.mark.parametrize("parts", [2, 5, 23])
def test_persistent_tail_parts_match_the_oracle(parts, monkeypatch):
    """The 44 tail tiles against 79 key tiles cut into 2, 5 or 23 parts (39-40 down to 3-4 key
    tiles each, 88 to 1012 runs: 23 parts is the most the workspace's tail room holds, 4 runs per
    CU plus one slot per tail tile), `parts` partials per tail row.  Rows of whole tiles, of tail
    tiles and of the ragged last tile of a head match the oracle, and the result is bitwise
    repeatable."""
    B, H, Sq, Skv, D = 1, 20, 3600, 5000, 128
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=43)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    lens, order = (2000, 3000), (1, 0)
    print("persistent, tail tiles in %d parts" % parts, flush=True)
    o, l = _run(qd, kd, vd, lens, order, "fused", monkeypatch, "1", tail=parts, out_dtype=torch.bfloat16)
    rows = sorted({0, 255, 256, 3583, 3584, 3599} | set(range(0, Sq, 89)))
    for h in (0, 17, 19):  # whole tiles only; tail from tile 256 (head 17, tile 1); tail only
        o_ref, l_ref = oracle.attention(q[:, h:h + 1, rows], k[:, h:h + 1], v[:, h:h + 1], 1 / math.sqrt(D))
        assert_parity(o[:, h:h + 1, rows], l[:, h:h + 1, rows], o_ref, l_ref,
                      what="persistent parts=%d head %d" % (parts, h))
    for _ in range(3):
        o2, l2 = _run(qd, kd, vd, lens, order, "fused", monkeypatch, "1", tail=parts, out_dtype=torch.bfloat16)
        assert torch.equal(o, o2) and torch.equal(l, l2)


def test_persistent_one_round_runs_one_workgroup_per_item(monkeypatch):
    """Three query tiles (one round): nothing to queue, the launch is one workgroup per item
    whether or not persistence is asked for."""
    B, H, Sq, Skv, D = 1, 3, 200, 5000, 128
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=45)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(D))
    o, l = _run(qd, kd, vd, (Skv,), None, "fused", monkeypatch, "1", tail=5, out_dtype=torch.bfloat16)
    assert_parity(o, l, o_ref, l_ref, what="one round, persistence asked")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_persistent_batches_strided_views_and_d64(D, out_dtype, monkeypatch):
    """Two batches with [B,S,H,D] storage for Q, K, V and O, 2 x 11 heads x 12 query tiles = 264
    (256 whole, 8 in the tail) against 5000 keys in two chunks, persistent, the tail tiles cut
    into 7 parts: every element against the oracle, and bitwise against one workgroup per item
    with one run of equal units per CU."""
    B, Sq, Skv, H = 2, 3000, 5000, 11
    rng = np.random.default_rng(7)
    qb, kb, vb = (synth.f32_to_bf16_bits(rng.standard_normal((B, S, H, D)).astype(np.float32))
                  for S in (Sq, Skv, Skv))
    qd, kd, vd = (to_device(x).permute(0, 2, 1, 3) for x in (qb, kb, vb))
    qh, kh, vh = (np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (qb, kb, vb))
    o_ref, l_ref = oracle.attention(qh, kh, vh, 1 / math.sqrt(D))
    print("persistent B=2 strided D=%d out %s" % (D, out_dtype), flush=True)

    def run(persist, tail):
        monkeypatch.setenv("LSDIT_DEBUG_PERSIST", persist)
        monkeypatch.setenv("LSDIT_DEBUG_TAIL", tail)
        out = torch.empty((B, Sq, H, D), dtype=out_dtype, device="cuda").permute(0, 2, 1, 3)
        o, l = A().shard_fwd(qd, kd, vd, (1700, 3300), (1, 0), mode="fused", out=out)
        torch.cuda.synchronize()
        assert o.data_ptr() == out.data_ptr()
        return o, l

    o, l = run("1", "7")
    assert_parity(o, l, o_ref, l_ref, what="persistent, 7 parts, B=2, strided, D=%d" % D)
    o_p, l_p = run("1", "ranges")
    o_s, l_s = run("0", "ranges")
    assert torch.equal(o_p, o_s) and torch.equal(l_p, l_s)
