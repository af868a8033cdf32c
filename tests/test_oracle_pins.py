"""Pins for the fp64 oracle against facts outside itself.

The pages print no worked example, so each check below is a closed form, an
invariant of softmax attention, a high-precision brute force on tiny inputs,
or an independent library (torch's CPU attention in fp64).  Together they
are chosen so that a dropped term, a wrong sign, a wrong index, a transposed
operand, a missing scale, a base-2 log or an overflow in the oracle fails at
least one of them.
"""
import math

import mpmath
import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rtol=1e-12, atol=1e-12):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


def _brute_mp(q, k, v, scale):
    """Pure-Python, 50-digit evaluation of the definition, for tiny shapes only."""
    mpmath.mp.dps = 50
    B, H, S, D = q.shape
    Skv = k.shape[2]
    o = np.zeros((B, H, S, D))
    lse = np.zeros((B, H, S))
    for b in range(B):
        for h in range(H):
            for i in range(S):
                s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(q[b, h, i, d])) * mpmath.mpf(float(k[b, h, j, d]))
                                                     for d in range(D)) for j in range(Skv)]
                w = [mpmath.exp(x) for x in s]
                tot = mpmath.fsum(w)
                lse[b, h, i] = float(mpmath.log(tot))
                for d in range(D):
                    o[b, h, i, d] = float(mpmath.fsum(w[j] * mpmath.mpf(float(v[b, h, j, d])) for j in range(Skv)) / tot)
    return o, lse


@pytest.mark.parametrize("S,Skv,D", [(1, 1, 1), (3, 5, 2), (8, 8, 4), (5, 7, 3)])
def test_brute_force_high_precision(S, Skv, D):
    r = _rng(S * 100 + Skv * 10 + D)
    q, k, v = r.standard_normal((1, 2, S, D)) * 2, r.standard_normal((1, 2, Skv, D)) * 2, r.standard_normal((1, 2, Skv, D))
    scale = 1 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale)
    o2, lse2 = _brute_mp(q, k, v, scale)
    _close(o, o2, rtol=1e-13, atol=1e-14)
    _close(lse, lse2, rtol=1e-13, atol=1e-14)


def test_single_key_returns_its_value_row():
    r = _rng(1)
    q, k, v = r.standard_normal((2, 3, 9, 16)), r.standard_normal((2, 3, 1, 16)), r.standard_normal((2, 3, 1, 16))
    o, lse = oracle.attention(q, k, v, 0.25)
    _close(o, np.broadcast_to(v, o.shape), rtol=0, atol=0)
    _close(lse, 0.25 * np.einsum("bhid,bhjd->bhi", q, k), rtol=1e-14)


def test_two_keys_closed_form():
    r = _rng(2)
    q, k, v = r.standard_normal((1, 2, 6, 8)) * 3, r.standard_normal((1, 2, 2, 8)), r.standard_normal((1, 2, 2, 8))
    sc = 0.3
    s = sc * np.einsum("bhid,bhjd->bhij", q, k)
    s0, s1 = s[..., 0], s[..., 1]
    lse_want = np.logaddexp(s0, s1)
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    o_want = sig(s0 - s1)[..., None] * v[:, :, None, 0, :] + sig(s1 - s0)[..., None] * v[:, :, None, 1, :]
    o, lse = oracle.attention(q, k, v, sc)
    _close(o, o_want)
    _close(lse, lse_want)


def test_zero_queries_give_uniform_weights():
    r = _rng(3)
    Skv = 37
    q = np.zeros((1, 2, 4, 8))
    k, v = r.standard_normal((1, 2, Skv, 8)), r.standard_normal((1, 2, Skv, 8))
    o, lse, p = oracle.attention(q, k, v, 0.7, want_p=True)
    _close(p, np.full(p.shape, 1.0 / Skv), rtol=1e-14, atol=0)
    _close(lse, np.full(lse.shape, math.log(Skv)), rtol=1e-15, atol=0)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape))


def test_softmax_rows_sum_to_one():
    r = _rng(4)
    q, k, v = r.standard_normal((1, 3, 20, 32)) * 2, r.standard_normal((1, 3, 300, 32)) * 2, r.standard_normal((1, 3, 300, 32))
    _, _, p = oracle.attention(q, k, v, 1 / math.sqrt(32), want_p=True)
    assert np.all(p >= 0)
    _close(p.sum(-1), np.ones(p.shape[:-1]), rtol=0, atol=1e-13)


def test_uniform_values_return_that_value():
    r = _rng(5)
    q, k = r.standard_normal((1, 2, 10, 16)) * 3, r.standard_normal((1, 2, 50, 16)) * 3
    row = r.standard_normal(16)
    v = np.broadcast_to(row, (1, 2, 50, 16)).copy()
    o, _ = oracle.attention(q, k, v, 0.25)
    _close(o, np.broadcast_to(row, o.shape), rtol=1e-13, atol=1e-14)


def test_one_hot_dominant_selects_single_value_row():
    # K_j = c e_j, Q_i = c e_pi(i): s_ij = c^2 scale delta(j, pi(i)).
    D = Skv = 16
    S = 16
    scale = 1 / math.sqrt(D)
    c = math.sqrt(50.0 / scale)
    perm = _rng(6).permutation(Skv)
    k = np.zeros((1, 1, Skv, D))
    q = np.zeros((1, 1, S, D))
    for j in range(Skv):
        k[0, 0, j, j] = c
    for i in range(S):
        q[0, 0, i, perm[i]] = c
    v = _rng(7).standard_normal((1, 1, Skv, D))
    o, lse = oracle.attention(q, k, v, scale)
    a = c * c * scale
    _close(o[0, 0], v[0, 0, perm], rtol=1e-15, atol=1e-15)
    _close(lse[0, 0], np.full(S, a + math.log1p((Skv - 1) * math.exp(-a))), rtol=1e-15, atol=0)


def test_planted_match_in_random_sign_keys_large_logits():
    # Keys are random +-1 vectors; query i is c times key pi(i).  The planted key beats any
    # other by at least 2*c*scale per differing sign, so it takes all the weight; logits
    # reach ~1280, which an implementation without the max shift would overflow on.
    r = _rng(8)
    D, Skv, S = 64, 300, 40
    scale = 1 / math.sqrt(D)
    k = r.choice([-1.0, 1.0], size=(1, 1, Skv, D))
    gram = k[0, 0] @ k[0, 0].T
    np.fill_diagonal(gram, -D)
    assert gram.max() <= D - 2
    c = 20.0 / scale
    pi = r.choice(Skv, size=S, replace=False)
    q = c * k[:, :, pi, :]
    v = r.standard_normal((1, 1, Skv, D))
    o, lse = oracle.attention(q, k, v, scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    _close(o[0, 0], v[0, 0, pi], rtol=0, atol=1e-12)
    _close(lse[0, 0], np.full(S, c * scale * D), rtol=1e-15, atol=0)


def test_affine_map_of_values_commutes():
    r = _rng(9)
    q, k, v = r.standard_normal((1, 2, 12, 16)), r.standard_normal((1, 2, 40, 16)), r.standard_normal((1, 2, 40, 16))
    o, lse = oracle.attention(q, k, v, 0.25)
    o2, lse2 = oracle.attention(q, k, -2.5 * v + 0.75, 0.25)
    _close(o2, -2.5 * o + 0.75)
    _close(lse2, lse, rtol=0, atol=0)


def test_joint_key_value_permutation_invariance():
    r = _rng(10)
    q, k, v = r.standard_normal((1, 2, 12, 16)), r.standard_normal((1, 2, 40, 16)), r.standard_normal((1, 2, 40, 16))
    perm = r.permutation(40)
    o, lse = oracle.attention(q, k, v, 0.25)
    o2, lse2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.25)
    _close(o2, o)
    _close(lse2, lse)
    # permuting the values alone must change the output
    o3, _ = oracle.attention(q, k, v[:, :, perm], 0.25)
    assert np.max(np.abs(o3 - o)) > 1e-3


def test_key_shift_moves_lse_only():
    r = _rng(11)
    q, k, v = r.standard_normal((1, 2, 12, 16)), r.standard_normal((1, 2, 40, 16)), r.standard_normal((1, 2, 40, 16))
    u = r.standard_normal(16)
    o, lse = oracle.attention(q, k, v, 0.25)
    o2, lse2 = oracle.attention(q, k + u, v, 0.25)
    _close(o2, o, rtol=1e-11, atol=1e-12)
    _close(lse2, lse + 0.25 * np.einsum("bhid,d->bhi", q, u), rtol=1e-12, atol=1e-12)


def test_torch_cpu_attention_agrees():
    torch = pytest.importorskip("torch")
    r = _rng(12)
    q, k, v = r.standard_normal((2, 3, 33, 64)), r.standard_normal((2, 3, 70, 64)), r.standard_normal((2, 3, 70, 64))
    scale = 1 / 8.0
    o, lse = oracle.attention(q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
    lt = torch.logsumexp(scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous()), dim=-1).numpy()
    _close(o, ot, rtol=1e-11, atol=1e-12)
    _close(lse, lt, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("lens,order", [
    ((64, 64, 64, 64), (0, 1, 2, 3)),
    ((30, 0, 97, 1, 128), (4, 2, 0, 3, 1)),
    ((100, 156), (1, 0)),
    ((256,), (0,)),
])
def test_chunk_partials_merge_to_unchunked(lens, order):
    r = _rng(13)
    q, k, v = r.standard_normal((1, 2, 24, 32)) * 2, r.standard_normal((1, 2, 256, 32)) * 2, r.standard_normal((1, 2, 256, 32))
    o, lse = oracle.attention(q, k, v, 0.2)
    parts = oracle.chunk_partials(q, k, v, 0.2, lens)
    om, lm = oracle.lse_merge([parts[c][0] for c in order], [parts[c][1] for c in order])
    _close(om, o)
    _close(lm, lse)
    # ring-style online merge, two at a time, in the same order
    acc_o, acc_l = parts[order[0]]
    for c in order[1:]:
        acc_o, acc_l = oracle.lse_merge([acc_o, parts[c][0]], [acc_l, parts[c][1]])
    _close(acc_o, o)
    _close(acc_l, lse)


def test_empty_key_range_and_merge_edges():
    r = _rng(14)
    q, k, v = r.standard_normal((1, 1, 5, 8)), r.standard_normal((1, 1, 16, 8)), r.standard_normal((1, 1, 16, 8))
    oe, le = oracle.attention(q, k, v, 0.5, kv_range=(7, 7))
    assert np.all(oe == 0) and np.all(le == -np.inf)
    o, lse = oracle.attention(q, k, v, 0.5)
    # one part: identity; with an empty part: identity; all empty: O = 0, LSE = -inf, no NaN
    o1, l1 = oracle.lse_merge([o], [lse])
    _close(o1, o, rtol=0, atol=0)
    _close(l1, lse, rtol=0, atol=0)
    o2, l2 = oracle.lse_merge([oe, o, oe], [le, lse, le])
    _close(o2, o, rtol=1e-15, atol=0)
    _close(l2, lse, rtol=0, atol=0)
    o3, l3 = oracle.lse_merge([oe, oe], [le, le])
    assert np.all(o3 == 0) and np.all(l3 == -np.inf)


def test_stored_dtypes_widen_exactly():
    r = _rng(15)
    import synth
    q64 = r.standard_normal((1, 2, 9, 16))
    k64 = r.standard_normal((1, 2, 30, 16))
    v64 = r.standard_normal((1, 2, 30, 16))
    qb, kb, vb = (synth.f32_to_bf16_bits(x.astype(np.float32)) for x in (q64, k64, v64))
    ob, lb = oracle.attention(qb, kb, vb, 0.25)
    qw, kw, vw = (synth.bf16_bits_to_f32(x).astype(np.float64) for x in (qb, kb, vb))
    ow, lw = oracle.attention(qw, kw, vw, 0.25)
    assert np.array_equal(ob, ow) and np.array_equal(lb, lw)
    of, lf = oracle.attention(q64.astype(np.float32), k64.astype(np.float32), v64.astype(np.float32), 0.25)
    og, lg = oracle.attention(*(x.astype(np.float32).astype(np.float64) for x in (q64, k64, v64)), 0.25)
    assert np.array_equal(of, og) and np.array_equal(lf, lg)


def test_row_selection_matches_full_rows():
    r = _rng(16)
    q, k, v = r.standard_normal((1, 2, 40, 16)), r.standard_normal((1, 2, 33, 16)), r.standard_normal((1, 2, 33, 16))
    o, lse = oracle.attention(q, k, v, 0.25)
    rows = [0, 5, 39, 17]
    os_, ls_ = oracle.attention(q, k, v, 0.25, q_rows=rows)
    assert np.array_equal(os_, o[:, :, rows]) and np.array_equal(ls_, lse[:, :, rows])
    oz, lz = oracle.attention(q[:, :, :0], k, v, 0.25)
    assert oz.shape == (1, 2, 0, 16) and lz.shape == (1, 2, 0)


# ---- Ulysses re-layout: pinned by brute force over every index, by the exchange property the
# layout exists for, and by the round trip.

def test_ulysses_pack_brute_force_indices():
    rng = np.random.default_rng(3)
    B, H, S, D, n = 2, 6, 5, 4, 3
    x = rng.standard_normal((B, H, S, D))
    p = oracle.ulysses_pack(x, n)
    assert p.shape == (n, S, B, H // n, D)
    for j in range(n):
        for s in range(S):
            for b in range(B):
                for hq in range(H // n):
                    for d in range(D):
                        assert p[j, s, b, hq, d] == x[b, j * (H // n) + hq, s, d]


def test_ulysses_exchange_concatenates_rank_slices():
    """Rank r packs its sequence slice; rank j receives part j from every rank.  Concatenating
    those parts by source rank equals part j of packing the whole sequence at once."""
    rng = np.random.default_rng(4)
    B, H, S, D, n = 2, 8, 12, 4, 4
    x = rng.standard_normal((B, H, S, D)).astype(np.float32)
    whole = oracle.ulysses_pack(x, n)
    sl = S // n
    per_rank = [oracle.ulysses_pack(x[:, :, r * sl:(r + 1) * sl], n) for r in range(n)]
    for j in range(n):
        received = np.concatenate([per_rank[r][j] for r in range(n)], axis=0)  # [S, B, Hg, D]
        assert np.array_equal(received, whole[j])


def test_ulysses_round_trip_and_single_group():
    rng = np.random.default_rng(5)
    x = rng.integers(0, 2**16, size=(1, 4, 7, 8), dtype=np.uint16)  # bf16 bit patterns
    for n in (1, 2, 4):
        assert np.array_equal(oracle.ulysses_unpack(oracle.ulysses_pack(x, n)), x)
    # one group: the packed part is x with its S and H axes moved
    assert np.array_equal(oracle.ulysses_pack(x, 1)[0], np.transpose(x, (2, 0, 1, 3)))


# ---- FP8 (OCP E4M3) decoding of the oracle and encoding of the input generator.
# The values below are fixed by the E4M3 format definition (bias 7, 3 mantissa bits,
# subnormal step 2^-9, largest finite 1.75 * 2^8, 0x7F/0xFF NaN, no infinities).

E4M3_KNOWN = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
              0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x44: 3.0, 0x58: 16.0, 0x59: 18.0,
              0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0x81: -(2.0 ** -9), 0xB8: -1.0, 0xFE: -448.0}


def test_e4m3_decode_format_values():
    codes = np.array(sorted(E4M3_KNOWN), dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(got, np.array([E4M3_KNOWN[int(c)] for c in codes]))
    assert np.signbit(oracle.e4m3_decode(np.array([0x80], np.uint8))[0])
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    # every finite positive code decodes to a strictly larger value than the one before it
    pos = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0


def test_e4m3_encode_round_trip_and_ties_to_even():
    import synth
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(synth.f64_to_e4m3_bits(vals), codes)
    # midpoints of neighbouring codes round to the even code (even mantissa), and values
    # just off the midpoint round to the nearer code
    lo = np.arange(0, 0x7E, dtype=np.uint8)
    a, b = oracle.e4m3_decode(lo), oracle.e4m3_decode(lo + 1)
    mid = (a + b) / 2
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(synth.f64_to_e4m3_bits(mid), even)
    assert np.array_equal(synth.f64_to_e4m3_bits(np.nextafter(mid, 0)), lo)
    assert np.array_equal(synth.f64_to_e4m3_bits(np.nextafter(mid, 1e9)), lo + 1)
    assert np.array_equal(synth.f64_to_e4m3_bits(-mid), even | 0x80)
    with pytest.raises(ValueError):
        synth.f64_to_e4m3_bits(np.array([464.0 + 1e-9]))
    with pytest.raises(ValueError):
        synth.f64_to_e4m3_bits(np.array([np.inf]))


def test_e4m3_quantize_relative_error_and_range():
    import synth
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4096) * 3.0
    codes, descale = synth.e4m3_quantize(x)
    back = oracle.e4m3_decode(codes) * descale
    assert np.max(np.abs(oracle.e4m3_decode(codes))) == 448.0
    normal = np.abs(x) >= 2.0 ** -6 * descale
    # round-to-nearest with 3 mantissa bits: relative error at most 2^-4 in the normal range
    assert np.all(np.abs(back - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * (1 + 1e-12))
    assert np.all(np.abs(back - x)[~normal] <= 2.0 ** -10 * descale * (1 + 1e-12))


def test_attention_e4m3_is_attention_of_decoded_values():
    # small integer codes with power-of-two descales: the decoded inputs are exact, so the
    # fp8 entry must equal the plain attention on the same values
    rng = np.random.default_rng(6)
    q8, k8, v8 = (rng.choice(np.array([0x30, 0x38, 0x3C, 0x40, 0xB0, 0xB8, 0xC0], np.uint8), size=(1, 2, 5, 8))
                  for _ in range(3))
    o, lse = oracle.attention_e4m3(q8, k8, v8, 0.5, 2.0, 0.25, 0.3)
    qd, kd, vd = (oracle.e4m3_decode(x) * s for x, s in ((q8, 0.5), (k8, 2.0), (v8, 0.25)))
    s = np.einsum("bhid,bhjd->bhij", qd, kd) * 0.3
    w = np.exp(s - s.max(-1, keepdims=True))
    assert np.allclose(o, np.einsum("bhij,bhjd->bhid", w / w.sum(-1, keepdims=True), vd), rtol=1e-13, atol=1e-14)
    assert np.allclose(lse, np.log(w.sum(-1)) + s.max(-1), rtol=1e-13, atol=1e-14)
    o2, lse2 = oracle.attention_e4m3(q8, k8, v8, 0.5, 2.0, 0.25, 0.3, q_rows=[4, 1])
    assert np.array_equal(o2, o[:, :, [4, 1]]) and np.array_equal(lse2, lse[:, :, [4, 1]])
