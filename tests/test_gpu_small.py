"""GPU parity at sizes the oracle finishes in seconds: every output element is compared.

Shapes span several query tiles (128 rows) and key tiles (64 rows) and end in
ragged tails; edge cases cover empty chunks, -inf merges, strided layouts,
the D = 64 path, fp32 partial outputs and bitwise repeatability.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads
from parity_util import assert_parity, to_device, to_f64

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


def _inputs(B, H, Sq, Skv, D, kind=synth.KIND_BF16, seed=0, qk=1.0):
    q = synth.normal_rows(seed, 0, B, H, Sq, D, factor=qk, kind=kind)
    k = synth.normal_rows(seed, 1, B, H, Skv, D, factor=qk, kind=kind)
    v = synth.normal_rows(seed, 2, B, H, Skv, D, kind=kind)
    return q, k, v


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_chunk_fwd_all_elements(D, out):
    B, H, Sq, Skv = 1, 3, 1000, 1500   # 1000 = 7*128 + 104, 1500 = 23*64 + 28
    q, k, v = _inputs(B, H, Sq, Skv, D, qk=1.3)
    scale = 1 / math.sqrt(D)
    o_ref, l_ref = oracle.attention(q, k, v, scale)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    o, l = A().chunk_fwd(to_device(q), to_device(k), to_device(v), scale, out_dtype=od)
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, what="chunk_fwd D=%d out=%s" % (D, out))


@pytest.mark.parametrize("Sq,Skv", [(1, 1), (31, 63), (33, 65), (129, 130), (128, 64), (257, 1)])
def test_tails(Sq, Skv):
    q, k, v = _inputs(2, 2, Sq, Skv, 128, seed=3)
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(128))
    o, l = A().chunk_fwd(to_device(q), to_device(k), to_device(v))
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, what="tails Sq=%d Skv=%d" % (Sq, Skv))


def test_tiny_fp32_config_all_modes():
    w = workloads.TINY
    x = w.make_inputs()
    q, k, v = (to_device(x[n]) for n in "qkv")
    o_ref, l_ref = oracle.attention(x["q"], x["k"], x["v"], w.scale)
    plan = w.plan()
    for mode in ("nway", "online", "fused"):
        o, l = A().shard_fwd(q, k, v, plan.lens, plan.order, mode=mode)
        torch.cuda.synchronize()
        assert_parity(o, l, o_ref, l_ref, fp32=True, what="tiny fp32 %s" % mode)
    o, l = A().shard_fwd(q, k, v, (256,))
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, fp32=True, what="tiny fp32 unchunked")
    # each chunk's partial against the oracle's partial over the same keys
    parts = oracle.chunk_partials(x["q"], x["k"], x["v"], w.scale, plan.lens)
    off = 0
    gparts = []
    for (po, pl), n in zip(parts, plan.lens):
        o, l = A().chunk_fwd(q, k[:, :, off:off + n], v[:, :, off:off + n], w.scale)
        torch.cuda.synchronize()
        assert_parity(o, l, po, pl, fp32=True, what="tiny partial @%d" % off)
        gparts.append((o, l))
        off += n
    # the standalone merge fed the oracle's partials rounded to fp32
    po = [torch.from_numpy(p[0].astype(np.float32)).cuda() for p in parts]
    pl = [torch.from_numpy(p[1].astype(np.float32)).cuda() for p in parts]
    o, l = A().lse_merge(po, pl, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, fp32=True, what="merge of oracle partials")


@pytest.mark.parametrize("mode", ["nway", "online", "fused"])
def test_shard_modes_orders_and_empty_chunks(mode):
    B, H, Sq, D = 1, 2, 300, 128
    lens = (100, 0, 257, 1, 64, 0, 178)
    q, k, v = _inputs(B, H, Sq, sum(lens), D, seed=5, qk=1.2)
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(D))
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    for order in (None, (6, 5, 4, 3, 2, 1, 0), (2, 0, 6, 1, 4, 5, 3)):
        o, l = A().shard_fwd(qd, kd, vd, lens, order, mode=mode)
        torch.cuda.synchronize()
        assert_parity(o, l, o_ref, l_ref, what="shard %s order %s" % (mode, order))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode", ["fused", "nway"])
def test_max_chunks_random_lengths_and_order(dtype, mode):
    """64 chunks (the most one call takes): random lengths from 0 to 150 (tiles that end
    mid-chunk, chunks shorter than a tile, empty chunks) walked in a random order."""
    rng = np.random.default_rng(11)
    lens = tuple(int(x) for x in rng.integers(0, 151, size=64))
    order = tuple(int(x) for x in rng.permutation(64))
    B, H, Sq, D = 1, 2, 130, 64
    kind = synth.KIND_BF16 if dtype == "bf16" else synth.KIND_F32
    q, k, v = _inputs(B, H, Sq, sum(lens), D, kind=kind, seed=9)
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(D))
    o, l = A().shard_fwd(to_device(q), to_device(k), to_device(v), lens, order, mode=mode)
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, fp32=dtype == "fp32", what="64 chunks %s %s" % (dtype, mode))


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("Skv", [5000, 9000])
def test_balanced_tail_few_query_tiles(Skv, D):
    """Three query tiles against 79 or 141 key tiles: with the workspace, the fused schedule
    spreads the work over the CUs as runs of about one key tile (the fix-up then merges some 80
    partials per row); without it, one workgroup per query tile.  Both match the oracle."""
    B, H, Sq = 1, 3, 200
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=21)
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(D))
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    lens = (Skv // 3, Skv - Skv // 3)
    need = A().shard_workspace_size(B, H, Sq, D, len(lens), "fused")
    assert need > 0  # 3 query tiles leave the last round part-full
    for ws in (torch.empty(need, dtype=torch.uint8, device="cuda"), torch.empty(0, dtype=torch.uint8, device="cuda")):
        o, l = A().shard_fwd(qd, kd, vd, lens, (1, 0), mode="fused", workspace=ws)
        torch.cuda.synchronize()
        assert_parity(o, l, o_ref, l_ref, what="Skv %d workspace %d" % (Skv, ws.numel()))


def test_balanced_tail_spans_query_tiles():
    """300 query tiles (20 heads x 15, the last of each head 16 rows) against 79 key tiles in two
    chunks: 256 run whole, and the 44 of the tail as 256 runs of 13-14 key tiles, many crossing
    from one query tile into the next.  Rows of whole tiles, of tail tiles (first, crossing,
    last) and of the ragged last tiles match the oracle; the result also matches the run
    without the tail."""
    B, H, Sq, Skv, D = 1, 20, 3600, 5000, 128
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=23)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    lens, order = (2000, 3000), (1, 0)
    need = A().shard_workspace_size(B, H, Sq, D, 2, "fused")
    assert need > 0
    o, l = A().shard_fwd(qd, kd, vd, lens, order, mode="fused",
                         workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    o_dp, l_dp = A().shard_fwd(qd, kd, vd, lens, order, mode="fused",
                               workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    # query tile t of the 15 per head: head t // 15, rows 256 (t % 15) ..; tiles 256.. are the tail
    rows = sorted({0, 255, 256, 3583, 3584, 3599} | set(range(0, Sq, 97)))
    for h in (0, 17, 19):  # whole tiles only; tail from tile 256 (head 17, tile 1); tail only
        o_ref, l_ref = oracle.attention(q[:, h:h + 1, rows], k[:, h:h + 1], v[:, h:h + 1], 1 / math.sqrt(D))
        assert_parity(o[:, h:h + 1, rows], l[:, h:h + 1, rows], o_ref, l_ref, what="tail spans, head %d" % h)
    assert float((o.float() - o_dp.float()).abs().max()) <= 2e-2
    assert float((l - l_dp).abs().max()) <= 1e-3


KERNEL_RESCALE_LOG2 = 64.0  # the bf16 kernel's lazy-rescale threshold (log2 units)


def _reference_moves(q, k, D, Skv):
    """Host-side count, per query row, of the tiles after the first on which the lazy rule moves
    the row's reference (a tile's scaled row max above the reference, which then goes to that max
    plus the threshold), from fp64 scores of the bf16 inputs."""
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    kf = synth.bf16_bits_to_f32(k).astype(np.float64)
    s = np.einsum("bhqd,bhkd->bhqk", qf, kf) * (math.log2(math.e) / math.sqrt(D))
    ref = np.full(s.shape[:-1], -np.inf)
    moves = np.zeros(s.shape[:-1], dtype=int)
    for t in range(0, Skv, 64):
        m = s[..., t:t + 64].max(-1)
        mv = m > ref
        if t > 0:
            moves += mv
        ref = np.where(mv, m + KERNEL_RESCALE_LOG2, ref)
    return moves


@pytest.mark.parametrize("growth", [11, 90])
@pytest.mark.parametrize("D", [128, 64])
def test_rescale_on_every_tile(D, growth):
    """Key rows scaled up along the sequence.  growth 11: each 64-key tile's row max grows by
    about 10 (log2 units), so the weights climb through the lazy-rescale headroom (2^64) and the
    reference moves 1 to 3 times after the first tile; growth 90: the row max grows by about 80
    per tile, past the headroom, so the references of the rows of positive sign (about half)
    move on most tiles and the rescale of the output and row sums runs on nearly every tile, in
    every mode."""
    B, H, Sq, Skv = 1, 2, 300, 900
    q = synth.normal_rows(31, 0, B, H, Sq, D, kind=synth.KIND_F64)
    k = synth.normal_rows(31, 1, B, H, Skv, D, kind=synth.KIND_F64)
    v = synth.normal_rows(31, 2, B, H, Skv, D)
    # every element of a query row has one sign and every key element is positive, growing along
    # the keys; rows of negative sign keep their first tile's reference
    q = synth.f32_to_bf16_bits((np.sign(q.sum(-1, keepdims=True)) * np.abs(q)).astype(np.float32))
    k = synth.f32_to_bf16_bits((np.abs(k) * (0.05 + growth * np.arange(Skv) / 64.0)[None, None, :, None] /
                                math.sqrt(D)).astype(np.float32))
    moves = _reference_moves(q, k, D, Skv)
    if growth == 11:
        assert 1 <= moves.max() <= 3
    else:  # 13 tiles after the first: rows of positive sign (about half) move on 8 or more
        assert moves.max() == 13 and np.count_nonzero(moves >= 8) >= 0.4 * moves.size
    scale = 1 / math.sqrt(D)
    o_ref, l_ref = oracle.attention(q, k, v, scale)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o, l = A().chunk_fwd(qd, kd, vd, scale)
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, what="rescale growth %d D=%d" % (growth, D))
    for mode in ("fused", "nway", "online"):
        ws = torch.empty(max(A().shard_workspace_size(B, H, Sq, D, 3, mode), 1), dtype=torch.uint8, device="cuda")
        o, l = A().shard_fwd(qd, kd, vd, (300, 350, 250), (2, 0, 1), mode=mode, workspace=ws)
        torch.cuda.synchronize()
        assert_parity(o, l, o_ref, l_ref, what="rescale growth %d D=%d %s" % (growth, D, mode))


@pytest.mark.parametrize("D", [128, 64])
def test_lse_of_rows_dominated_by_one_key(D):
    """Each query row i has one planted key (key i, along q_i, with a score of 20 natural units;
    no other score of the row above 9 for D = 128, 14 for D = 64), which carries nearly all of
    the row's weight.  P.V and the
    row sum use the weights rounded to bf16, so the LSE would carry that key's rounding (up to
    2^-9 relative, about 1e-3 on average); the kernel's LSE takes the row's largest weight
    unrounded, so its error stays at fp32 level: 1e-4 on every row, in every mode (the key in
    one chunk of three, a balanced tail where there is one), while O stays within the bf16 gate."""
    B, H, Sq, Skv = 1, 2, 600, 900
    q64 = synth.normal_rows(61, 0, B, H, Sq, D, kind=synth.KIND_F64)
    k64 = synth.normal_rows(61, 1, B, H, Skv, D, kind=synth.KIND_F64)
    v = synth.normal_rows(61, 2, B, H, Skv, D)
    qn = q64 / np.linalg.norm(q64, axis=-1, keepdims=True)
    k64[:, :, :Sq] = 20.0 * math.sqrt(D) * qn / np.linalg.norm(q64, axis=-1, keepdims=True)
    q = synth.f32_to_bf16_bits(q64.astype(np.float32))
    k = synth.f32_to_bf16_bits(k64.astype(np.float32))
    scale = 1 / math.sqrt(D)
    o_ref, l_ref = oracle.attention(q, k, v, scale)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    runs = [("chunk", A().chunk_fwd(qd, kd, vd, scale))]
    for mode in ("fused", "nway", "online"):
        runs.append((mode, A().shard_fwd(qd, kd, vd, (300, 350, 250), (2, 0, 1), mode=mode)))
    torch.cuda.synchronize()
    for what, (o, l) in runs:
        err = float(np.abs(to_f64(l) - l_ref).max())
        print("dominant key, D=%d %s: LSE max-abs %.3g" % (D, what, err), flush=True)
        assert err <= 1e-4, (what, err)
        assert_parity(o, l, o_ref, l_ref, what="dominant key D=%d %s" % (D, what))


def test_bf16_chunk_partials_and_merge():
    B, H, Sq, D = 1, 2, 200, 128
    lens = (70, 130, 64)
    q, k, v = _inputs(B, H, Sq, sum(lens), D, seed=6)
    scale = 1 / math.sqrt(D)
    parts = oracle.chunk_partials(q, k, v, scale, lens)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    off, go, gl = 0, [], []
    for (po, pl), n in zip(parts, lens):
        o, l = A().chunk_fwd(qd, kd[:, :, off:off + n], vd[:, :, off:off + n], scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_parity(o, l, po, pl, what="bf16 partial @%d" % off)
        go.append(o)
        gl.append(l)
        off += n
    o_ref, l_ref = oracle.attention(q, k, v, scale)
    o, l = A().lse_merge(go, gl, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, what="merge of GPU partials")
    # ring-style in-place online merge: out aliases part 0
    acc_o, acc_l = go[0].clone(), gl[0].clone()
    for c in (1, 2):
        A().lse_merge([acc_o, go[c]], [acc_l, gl[c]], out=acc_o, lse=acc_l)
    torch.cuda.synchronize()
    assert_parity(acc_o, acc_l, o_ref, l_ref, what="in-place online merge")


def test_empty_chunk_and_minus_inf_merges():
    B, H, Sq, D = 1, 2, 50, 64
    q, k, v = _inputs(B, H, Sq, 40, D, seed=7)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o, l = A().chunk_fwd(qd, kd[:, :, :0], vd[:, :, :0], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))
    o1, l1 = A().chunk_fwd(qd, kd, vd, out_dtype=torch.float32)
    om, lm = A().lse_merge([o, o1, o], [l, l1, l], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(lm, l1)
    assert torch.allclose(om, o1, rtol=0, atol=1e-7)
    oe, le = A().lse_merge([o, o], [l, l], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(oe == 0) and torch.all(torch.isneginf(le)) and not torch.isnan(oe).any()
    # a plan whose chunks are all empty
    oz, lz = A().shard_fwd(qd, kd[:, :, :0], vd[:, :, :0], (0, 0), mode="nway")
    torch.cuda.synchronize()
    assert torch.all(oz == 0) and torch.all(torch.isneginf(lz))


def test_strided_bshd_views():
    B, S, H, D = 2, 333, 3, 128
    rng = np.random.default_rng(1)
    base = [synth.f32_to_bf16_bits(rng.standard_normal((B, S, H, D)).astype(np.float32)) for _ in range(3)]
    qd, kd, vd = (to_device(x).permute(0, 2, 1, 3) for x in base)  # [B,H,S,D] views of [B,S,H,D]
    out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    qh, kh, vh = (np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in base)
    o_ref, l_ref = oracle.attention(qh, kh, vh, 1 / math.sqrt(D))
    o, l = A().chunk_fwd(qd, kd, vd, out=out)
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, what="strided chunk_fwd")
    out2 = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    o, l = A().shard_fwd(qd, kd, vd, (100, 233), (1, 0), mode="fused", out=out2)
    torch.cuda.synchronize()
    assert_parity(o, l, o_ref, l_ref, what="strided shard_fwd")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_balanced_tail_batches_and_strided_views(out_dtype):
    """Two batches, [B,S,H,D] storage for Q, K, V and O, 5000 keys in two chunks: the 12 query
    tiles run as 256 tail runs whose fix-up writes through the strided output."""
    B, Sq, Skv, H, D = 2, 300, 5000, 3, 128
    rng = np.random.default_rng(5)
    qb, kb, vb = (synth.f32_to_bf16_bits(rng.standard_normal((B, S, H, D)).astype(np.float32))
                  for S in (Sq, Skv, Skv))
    qd, kd, vd = (to_device(x).permute(0, 2, 1, 3) for x in (qb, kb, vb))
    qh, kh, vh = (np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (qb, kb, vb))
    o_ref, l_ref = oracle.attention(qh, kh, vh, 1 / math.sqrt(D))
    assert A().shard_workspace_size(B, H, Sq, D, 2, "fused") > 0
    out = torch.empty((B, Sq, H, D), dtype=out_dtype, device="cuda").permute(0, 2, 1, 3)
    o, l = A().shard_fwd(qd, kd, vd, (1700, 3300), (1, 0), mode="fused", out=out)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    assert_parity(o, l, o_ref, l_ref, what="tail, B=2, strided, out %s" % out_dtype)


def test_nonfinite_inputs_through_the_tail():
    """One query tile against 79 key tiles runs as 79 one-tile runs merged by the fix-up: a NaN in
    V still reaches every output of its column (and only that column), and a NaN in K, which
    makes that key's score NaN in every row, every output and LSE."""
    D = 128
    q, k, v = _inputs(1, 1, 64, 5000, D, seed=10)
    assert A().shard_workspace_size(1, 1, 64, D, 1, "fused") > 0
    v[0, 0, 3000, 7] = 0x7FC0
    o, l = A().shard_fwd(to_device(q), to_device(k), to_device(v), (5000,), None, mode="fused",
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isnan(o[0, 0, :, 7]).all() and torch.isfinite(l).all()
    assert torch.isfinite(o[0, 0, :, :7]).all() and torch.isfinite(o[0, 0, :, 8:]).all()
    v[0, 0, 3000, 7] = v[0, 0, 3001, 7]
    k[0, 0, 2000, 3] = 0x7FC0
    o, l = A().shard_fwd(to_device(q), to_device(k), to_device(v), (5000,), None, mode="fused",
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(l).all()


def test_uniform_values_and_determinism():
    B, H, Sq, Skv, D = 1, 2, 256, 700, 128
    q, k, _ = _inputs(B, H, Sq, Skv, D, seed=8, qk=1.5)
    row = synth.f32_to_bf16_bits(np.linspace(-2, 2, D).astype(np.float32))
    v = np.broadcast_to(row, (B, H, Skv, D)).copy()
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o, l = A().chunk_fwd(qd, kd, vd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = synth.bf16_bits_to_f32(row).astype(np.float64)
    err = np.abs(to_f64(o) - want).max()
    assert err <= 2e-2 * np.abs(want).max(), err
    o2, l2 = A().chunk_fwd(qd, kd, vd, out_dtype=torch.float32)
    o3, l3 = A().shard_fwd(qd, kd, vd, (300, 400), mode="fused", out_dtype=torch.float32)
    o4, l4 = A().shard_fwd(qd, kd, vd, (300, 400), mode="fused", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(l, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


def test_noop_and_nonfinite_inputs():
    D = 128
    qd = torch.empty((1, 2, 0, D), dtype=torch.bfloat16, device="cuda")
    kd = torch.zeros((1, 2, 10, D), dtype=torch.bfloat16, device="cuda")
    o, l = A().chunk_fwd(qd, kd, kd)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, D)
    q, k, v = _inputs(1, 1, 64, 64, D, seed=9)
    v[0, 0, 5, 7] = 0x7FC0  # a NaN in V propagates to every output of that column
    o, l = A().chunk_fwd(to_device(q), to_device(k), to_device(v), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isnan(o[0, 0, :, 7]).all() and torch.isfinite(l).all()


@pytest.mark.parametrize("mode", ["fused", "online", "nway"])
def test_nan_query_row_every_schedule(mode):
    """A NaN in one query row makes every score of that row NaN, so its O and LSE are NaN, as in
    one pass over all keys; every other row stays finite and at parity.  One query tile against
    79 key tiles in two chunks: the fused schedule runs it as the balanced tail (the fix-up
    merges some 80 partials per row), and the online and n-way schedules merge per-chunk
    partials: neither merge may turn the NaN row into the 'no keys' result O = 0, LSE = -inf."""
    D = 128
    q, k, v = _inputs(1, 1, 64, 5000, D, seed=12)
    q[0, 0, 17, 5] = 0x7FC0
    keep = [r for r in range(64) if r != 17]
    o_ref, l_ref = oracle.attention(q[:, :, keep], k, v, 1 / math.sqrt(D))
    o1, l1 = A().chunk_fwd(to_device(q), to_device(k), to_device(v), out_dtype=torch.float32)
    o, l = A().shard_fwd(to_device(q), to_device(k), to_device(v), (1700, 3300), (1, 0), mode=mode,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    for oo, ll, what in ((o1, l1, "one pass"), (o, l, mode)):
        assert torch.isnan(oo[0, 0, 17]).all() and torch.isnan(ll[0, 0, 17]), what
        assert_parity(oo[:, :, keep], ll[:, :, keep], o_ref, l_ref, what="NaN query row, other rows, " + what)


@pytest.mark.parametrize("Skv", [1000, 63, 5000])
def test_rows_past_the_keys_are_not_read(Skv):
    """K and V are views of the first Skv rows of longer buffers whose rows past Skv hold NaN.
    The last, partial key tile and the tiles fetched past the last chunk must read those rows
    as zeros (a NaN V row times P = 0 would poison every output): the results stay finite and
    at parity, for one chunk and for the fused schedule with and without the balanced tail."""
    D, B, H, Sq = 128, 1, 2, 300
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=13)
    pad = 320  # more rows than any prefetch reaches past the end: every read stays in the buffer
    kb = np.full((B, H, Skv + pad, D), 0x7FC0, np.uint16)
    vb = np.full((B, H, Skv + pad, D), 0x7FC0, np.uint16)
    kb[:, :, :Skv] = k
    vb[:, :, :Skv] = v
    kd, vd = to_device(kb)[:, :, :Skv], to_device(vb)[:, :, :Skv]
    qd = to_device(q)
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(D))
    lens = (Skv // 3, Skv - Skv // 3)
    runs = [("chunk", lambda: A().chunk_fwd(qd, kd, vd)),
            ("fused", lambda: A().shard_fwd(qd, kd, vd, lens, (1, 0), mode="fused")),
            ("fused, no workspace", lambda: A().shard_fwd(qd, kd, vd, lens, (1, 0), mode="fused",
                                                          workspace=torch.empty(0, dtype=torch.uint8,
                                                                                device="cuda")))]
    for what, fn in runs:
        o, l = fn()
        torch.cuda.synchronize()
        assert_parity(o, l, o_ref, l_ref, what="NaN rows past Skv=%d, %s" % (Skv, what))


def test_side_stream_with_allocations_on_the_current_stream():
    """shard_fwd on a side stream allocates its workspace and outputs on the current stream; the
    binding records their use on the side stream, so buffers the current stream allocates and
    fills meanwhile never reuse that memory while the kernels still write it."""
    D, B, H, Sq, Skv = 128, 1, 3, 600, 9000
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=14)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(D), q_rows=[0, 299, 599])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    results = []
    for mode in ("online", "fused", "nway"):
        o, l = A().shard_fwd(qd, kd, vd, (3000, 6000), (1, 0), mode=mode, stream=side)
        results.append((mode, o, l))
        # the current stream allocates and fills memory while the side stream still runs
        junk = [torch.full((1 << 22,), float("nan"), device="cuda") for _ in range(8)]
        del junk
    torch.cuda.synchronize()
    for mode, o, l in results:
        assert_parity(o[:, :, [0, 299, 599]], l[:, :, [0, 299, 599]], o_ref, l_ref, what="side stream " + mode)


def test_determinism_through_the_balanced_tail():
    """A fixed plan is bitwise repeatable on the tail path too: runs of key tiles, their fp32
    partials and the fix-up's merge order are fixed (no atomics)."""
    D, B, H, Sq, Skv = 128, 1, 20, 3600, 5000
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=15)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    assert A().shard_workspace_size(B, H, Sq, D, 2, "fused") > 0
    o, l = A().shard_fwd(qd, kd, vd, (2000, 3000), (1, 0), mode="fused", out_dtype=torch.float32)
    for _ in range(3):
        o2, l2 = A().shard_fwd(qd, kd, vd, (2000, 3000), (1, 0), mode="fused", out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(l, l2)


@pytest.mark.parametrize("order", ["reverse", "rotate"])
def test_workgroup_order_does_not_change_results(order, monkeypatch):
    """Dispatching the forward kernels' logical workgroups in another order (the library's debug
    aid LSDIT_DEBUG_WG_ORDER: reversed, or rotated by half the grid) gives bitwise the same O and
    LSE: whole query tiles and the balanced tail's runs write disjoint rows and slots, nothing is
    accumulated across workgroups, and the fix-up merges in a fixed order.  The fused schedule
    with the tail (300 query tiles: 256 whole, 44 as runs), the per-chunk schedules, and the FP8
    variant with its tail."""
    D, B, H, Sq, Skv = 128, 1, 20, 3600, 5000
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=16)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    x8 = {n: synth.e4m3_quantize(synth.normal_rows(17, i, 1, 3, 200, D, kind=synth.KIND_F32))
          for i, n in enumerate("qkv")}
    c8 = {n: torch.from_numpy(x8[n][0]).cuda() for n in "qkv"}

    def runs():
        out = []
        for mode in ("fused", "online", "nway"):
            out.append(A().shard_fwd(qd, kd, vd, (2000, 3000), (1, 0), mode=mode, out_dtype=torch.float32))
        out.append(A().chunk_fwd_fp8(c8["q"], c8["k"], c8["v"], x8["q"][1], x8["k"][1], x8["v"][1], 0.1,
                                     out_dtype=torch.float32))
        torch.cuda.synchronize()
        return out

    monkeypatch.delenv("LSDIT_DEBUG_WG_ORDER", raising=False)
    ref = runs()
    monkeypatch.setenv("LSDIT_DEBUG_WG_ORDER", order)
    got = runs()
    for (o, l), (o2, l2), what in zip(ref, got, ("fused", "online", "nway", "fp8")):
        assert torch.equal(o, o2) and torch.equal(l, l2), "%s, order %s" % (what, order)
