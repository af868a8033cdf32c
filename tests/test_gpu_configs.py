"""GPU parity at the five workload shapes, in the launch configuration the bench times.

The image shape (4,608 tokens) is checked against the oracle on every row.  At
44,160 keys the oracle checks sampled query rows one by one (tile edges near
both ends, rank boundaries, the last rows and seeded random rows, in every
head): at least 8,192 (row, head) pairs per workload.  Properties that hold at
any size are checked on every row: all chunkings and merge schedules agree
with the unchunked result, and the ring share equals the matching rows of the
full sequence.  (bench.py --full-check compares every row of the full
sequence with the oracle.)
"""
import numpy as np
import pytest
import torch

import oracle
from synth import workloads
from parity_util import BF16_MAX_ABS, BF16_MEAN_ABS, assert_parity, errors, to_device, to_f64

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


class Case:
    """A workload's inputs on the device and the oracle's result on its checked rows (every row
    when n_random is None)."""

    def __init__(self, w, n_random=48):
        print("[case] %s: generating inputs" % w.name, flush=True)
        self.w = w
        self.host = w.make_inputs()
        self.dev = {n: to_device(x) for n, x in self.host.items()}
        bounds = [w.Sq * i // 8 for i in range(1, 8)]
        if n_random is None:
            self.rows = np.arange(w.Sq, dtype=np.int64)
        else:
            self.rows = workloads.sample_rows(w.Sq, bounds, n_random=n_random)
        print("[case] %s: oracle on %d rows x %d heads" % (w.name, len(self.rows), w.H), flush=True)
        self.o_ref, self.l_ref = oracle.attention(self.host["q"], self.host["k"], self.host["v"], w.scale,
                                                  q_rows=None if n_random is None else self.rows)

    def run(self, plan_name=None, mode="fused", out_dtype=None):
        p = self.w.plan(plan_name)
        o, l = A().shard_fwd(self.dev["q"], self.dev["k"], self.dev["v"], p.lens, p.order, mode=mode,
                             out_dtype=out_dtype)
        torch.cuda.synchronize()
        return o, l

    def check(self, o, l, what):
        if len(self.rows) == self.w.Sq:
            return assert_parity(o, l, self.o_ref, self.l_ref, what=what)
        return assert_parity(o[:, :, self.rows], l[:, :, self.rows], self.o_ref, self.l_ref, what=what)

    def free(self):
        self.dev = None
        torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def image_dit():
    c = Case(workloads.IMAGE_DIT, n_random=None)  # every row (about 0.26 fp64 TFLOP)
    yield c
    c.free()


@pytest.fixture(scope="module")
def ring_share():
    c = Case(workloads.RING_SHARE, n_random=500)  # >= 512 rows x 16 heads
    yield c
    c.free()


@pytest.fixture(scope="module")
def ulysses():
    c = Case(workloads.ULYSSES_SHARE, n_random=2100)  # >= 2,048 rows x 4 heads
    yield c
    c.free()


@pytest.fixture(scope="module")
def full_seq():
    c = Case(workloads.FULL_SEQUENCE, n_random=500)  # >= 512 rows x 16 heads
    yield c
    c.free()


def test_image_dit(image_dit):
    o, l = image_dit.run()
    image_dit.check(o, l, "image_dit")


@pytest.mark.parametrize("mode", ["fused", "online", "nway"])
def test_ring_share_modes(ring_share, mode):
    o, l = ring_share.run(mode=mode)
    ring_share.check(o, l, "ring_share %s" % mode)


def test_ring_share_chunk_partials(ring_share):
    c = ring_share
    plan = c.w.plan()
    off = 0
    for ci, n in enumerate(plan.lens):
        o, l = A().chunk_fwd(c.dev["q"], c.dev["k"][:, :, off:off + n], c.dev["v"][:, :, off:off + n], c.w.scale,
                             out_dtype=torch.float32)
        torch.cuda.synchronize()
        po, pl = oracle.attention(c.host["q"], c.host["k"], c.host["v"], c.w.scale, kv_range=(off, off + n),
                                  q_rows=c.rows)
        assert_parity(o[:, :, c.rows], l[:, :, c.rows], po, pl, what="ring partial chunk %d" % ci)
        off += n


def test_ring_share_other_rank():
    w = workloads.ring_share(rank=5)
    c = Case(w, n_random=16)
    o, l = c.run()
    c.check(o, l, "ring_share rank 5")
    c.free()


def test_ulysses_share(ulysses):
    o, l = ulysses.run()
    ulysses.check(o, l, "ulysses_share")


PLANS = ["chunks1", "chunks2", "chunks4", "chunks8", "ragged", "ring8"]


def _all_rows_close(o, l, o1, l1, what, host, scale, n_worst=4):
    """Two fp32 results of the same problem, compared on every row.

    Each result is within the bf16 gate of the oracle (max-abs 2e-2, mean-abs 2e-3) on the
    sampled rows, so on any row two of them can differ by up to twice the gate; that is the
    all-rows bound.  The rows where they differ most are then checked one by one against the
    oracle, each result to the gate itself.
    """
    do = (o.double() - o1.double()).abs()
    dl = (l.double() - l1.double()).abs()
    r = (do.max().item(), do.mean().item(), dl.max().item(), dl.mean().item())
    print("  %s all rows vs reference run: O max/mean %.3g/%.3g LSE max/mean %.3g/%.3g" % ((what,) + r), flush=True)
    assert r[0] <= 2 * BF16_MAX_ABS and r[1] <= 2 * BF16_MEAN_ABS, r
    assert r[2] <= 2 * BF16_MAX_ABS and r[3] <= 2 * BF16_MEAN_ABS, r
    per_row = do.amax(dim=(0, 1, 3))  # worst disagreement of each sequence row over heads
    rows = sorted(torch.topk(per_row, min(n_worst, per_row.numel())).indices.tolist())
    o_ref, l_ref = oracle.attention(host["q"], host["k"], host["v"], scale, q_rows=rows)
    assert_parity(o[:, :, rows], l[:, :, rows], o_ref, l_ref, what="  %s, rows %s" % (what, rows))
    assert_parity(o1[:, :, rows], l1[:, :, rows], o_ref, l_ref, what="  reference run, rows %s" % rows)


def _bf16_is_rounded_f32(o_bf16, o_f32, l_bf16run, l_f32run):
    """The bf16 output is the round-to-nearest-even of the fp32 value the same plan computes."""
    assert torch.equal(o_bf16, o_f32.to(torch.bfloat16))
    assert torch.equal(l_bf16run, l_f32run)


def test_full_sequence_plans_agree(full_seq):
    o1, l1 = full_seq.run("chunks1")
    full_seq.check(o1, l1, "full chunks1")
    o1f, l1f = full_seq.run("chunks1", out_dtype=torch.float32)
    _bf16_is_rounded_f32(o1, o1f, l1, l1f)
    for name in PLANS[1:]:
        for mode in (("fused", "online", "nway") if name == "chunks8" else ("fused",)):
            o, l = full_seq.run(name, mode)
            full_seq.check(o, l, "full %s %s" % (name, mode))
            of, lf = full_seq.run(name, mode, out_dtype=torch.float32)
            _bf16_is_rounded_f32(o, of, l, lf)
            _all_rows_close(of, lf, o1f, l1f, "%s %s" % (name, mode), full_seq.host, full_seq.w.scale)
            del o, l, of, lf


def test_ring_share_equals_full_sequence_rows(ring_share):
    # same seed, no outliers in the ring share: compare against a full-sequence run without outliers
    w = workloads.Workload("full_no_outliers", 1, 16, 44160, 44160, 128, "bf16",
                           plans={"c1": workloads.ChunkPlan((44160,))}, default_plan="c1")
    x = w.make_inputs()
    assert np.array_equal(x["k"], ring_share.host["k"])
    qd = to_device(x["q"])
    o, l = A().shard_fwd(qd, ring_share.dev["k"], ring_share.dev["v"], (44160,), out_dtype=torch.float32)
    o_r, l_r = ring_share.run(out_dtype=torch.float32)
    torch.cuda.synchronize()
    _all_rows_close(o_r, l_r, o[:, :, :5520], l[:, :, :5520], "ring share vs full rows", ring_share.host,
                    ring_share.w.scale)
