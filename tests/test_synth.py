"""Seeded input generator: published known answers, rounding, counter addressing."""
import math
import os

import numpy as np

import synth
from synth import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        w = [int(x, 16) for x in line.split()]
        assert synth.philox4x32_10(w[0:4], w[4:6]) == w[6:10]
        n += 1
    assert n == 3


def test_raw_words_follow_blocks():
    # word w of stream (seed, tid) is output (w mod 4) of block {w/4, 0, tid, 0} under key {seed, 0}
    raw = synth.raw_u32(5, 2, 3, 9)
    for i, w in enumerate(range(3, 12)):
        blk = synth.philox4x32_10([w // 4, 0, 2, 0], [5, 0])
        assert raw[i] == blk[w % 4]


def test_box_muller_element_mapping():
    B, H, S, D = 1, 2, 3, 8
    z = synth.normal_rows(11, synth.TID_V, B, H, S, D, kind=synth.KIND_F64).reshape(-1)
    raw = synth.raw_u32(11, synth.TID_V, 0, z.size).astype(np.float64)
    u = (raw + 0.5) / 2.0 ** 32
    for e in range(z.size):
        p = (e // 2) * 2
        r = math.sqrt(-2.0 * math.log(u[p]))
        t = 2.0 * math.pi * u[p + 1]
        want = r * math.cos(t) if e % 2 == 0 else r * math.sin(t)
        assert abs(z[e] - want) <= 1e-12 * max(1.0, abs(want))


def test_row_slices_regenerate_independently():
    full = synth.normal_rows(0, synth.TID_Q, 2, 3, 50, 16, kind=synth.KIND_BF16)
    part = synth.normal_rows(0, synth.TID_Q, 2, 3, 50, 16, 17, 33, kind=synth.KIND_BF16)
    assert np.array_equal(full[:, :, 17:33], part)


def test_rounding_chain_and_factors():
    z = synth.normal_rows(3, 1, 1, 2, 40, 32, kind=synth.KIND_F64)
    f32 = synth.normal_rows(3, 1, 1, 2, 40, 32, factor=1.5, kind=synth.KIND_F32)
    assert np.array_equal(f32, (1.5 * z).astype(np.float32))
    bf = synth.normal_rows(3, 1, 1, 2, 40, 32, factor=1.5, kind=synth.KIND_BF16)
    assert np.array_equal(bf, synth.f32_to_bf16_bits((1.5 * z).astype(np.float32)))
    rf = np.ones(40)
    rf[[3, 7]] = 8.0
    bo = synth.normal_rows(3, 1, 1, 2, 40, 32, row_factor=rf, kind=synth.KIND_F32)
    assert np.array_equal(bo, (z * rf[None, None, :, None]).astype(np.float32))


def test_bf16_round_to_nearest_even_bit_patterns():
    cases = {
        0x3F800000: 0x3F80,  # 1.0 exact
        0x3F808000: 0x3F80,  # tie, even stays
        0x3F818000: 0x3F82,  # tie, odd rounds up
        0x3F808001: 0x3F81,  # just above the tie
        0x3F807FFF: 0x3F80,  # just below the tie
        0xBF818000: 0xBF82,  # negative tie to even
        0x7F7FFFFF: 0x7F80,  # max finite rounds to +inf
        0x00000001: 0x0000,  # tiny denormal to zero
        0x7F800000: 0x7F80,  # +inf
    }
    src = np.array(list(cases), dtype=np.uint32).view(np.float32)
    got = synth.f32_to_bf16_bits(src)
    assert [int(x) for x in got] == list(cases.values())
    for bits, want in cases.items():
        f = np.array([bits], dtype=np.uint32).view(np.float32)[0]
        assert synth._load().synth_f32_to_bf16(float(f)) == want
    nan = np.array([0x7FC00001], dtype=np.uint32).view(np.float32)
    assert np.isnan(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(nan)))[0]


def test_normal_statistics():
    z = synth.normal_rows(0, 0, 1, 1, 512, 256, kind=synth.KIND_F64).reshape(-1)
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    assert abs(np.mean(np.abs(z) < 1.0) - 0.6826894921) < 0.01


def test_workload_recipes():
    assert workloads.ragged_chunks(44160, 5000, 1000) == [5000, 6000, 7000, 8000, 9000, 9160]
    assert workloads.ring_order(0, 8) == [0, 7, 6, 5, 4, 3, 2, 1]
    assert workloads.ring_order(3, 8) == [3, 2, 1, 0, 7, 6, 5, 4]
    for w in workloads.WORKLOADS.values():
        for plan in w.plans.values():
            assert sum(plan.lens) == w.Skv
            if plan.order is not None:
                assert sorted(plan.order) == list(range(len(plan.lens)))
    fs = workloads.FULL_SEQUENCE
    pos = fs.outlier_positions()
    assert len(pos) == 441 and len(set(pos.tolist())) == 441 and pos.min() >= 0 and pos.max() < 44160
    assert workloads.RING_SHARE.Sq == 5520 and workloads.RING_SHARE.q_row_lo == 0
    assert abs(fs.flops - 15.975e12) < 0.001e12


def test_tiny_inputs_shape_and_ring_slice():
    t = workloads.TINY.make_inputs()
    assert t["q"].dtype == np.float32 and t["q"].shape == (1, 2, 256, 64)
    # the ring rank's query slice is the same rows of the full-sequence draw
    w = workloads.ring_share(rank=5)
    q5 = synth.normal_rows(0, synth.TID_Q, 1, 16, 44160, 128, 5 * 5520, 5 * 5520 + 7)
    qs = synth.normal_rows(0, synth.TID_Q, 1, 16, w.s_full, 128, w.q_row_lo, w.q_row_lo + 7)
    assert np.array_equal(q5, qs)
