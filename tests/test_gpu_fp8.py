"""GPU parity of the FP8 (OCP E4M3) variant, attn_chunk_fwd_fp8, against the oracle on the
decoded inputs.

Tolerance, from the kernel's arithmetic.  Products of two E4M3 values are exact in fp32 and
the scores are fp32 sums, so the one rounding that matters is that of each probability to
E4M3 before P.V.  The kernel stores p' = 2^5 p, where p = 2^(x - m) uses a reference m at
most 3 (log2 units) below the row max: every key whose normalised probability P_j / P_max is
at least 2^-11 has p' >= 2^-6, a normal E4M3 number, rounded with relative error <= 2^-4;
smaller ones are rounded with absolute error <= 2^-10 in p', i.e. <= 2^-15 in p, against a
row sum of p that is at least 1 / P_max.  So per element

    |O - O_ref| <= 2^-4 A + 2^-15 P_max S + 2^-8 |O_ref| + 1e-6

with A = sum_j P_j |v_j| (attention of |V|), S = sum over keys with P_j < 2^-11 P_max of
|v_j|, and 2^-8 |O_ref| covering the bf16 store; the row sum adds the same rounded values,
so |LSE - LSE_ref| <= ln(1 + 2^-4) + 2^-15 P_max N_small + 1e-6.  Round-to-nearest-even errors
are unbiased, so on average the O error is far below the bound: its mean must stay under
2^-6 of the mean of A.  The LSE of a row that one key dominates carries that key's rounding
error undiminished (the reference may sit up to 3 below its score, so its 2^5 p is not a power
of two in general); the mean relative error of round-to-nearest with 3 mantissa bits is at
most 2^-5, which bounds the mean LSE error.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads
from parity_util import to_f64

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


def _codes_to_device(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _quantized(B, H, Sq, Skv, D=128, seed=0, qk=1.0):
    src = {"q": synth.normal_rows(seed, 0, B, H, Sq, D, factor=qk, kind=synth.KIND_F32),
           "k": synth.normal_rows(seed, 1, B, H, Skv, D, factor=qk, kind=synth.KIND_F32),
           "v": synth.normal_rows(seed, 2, B, H, Skv, D, kind=synth.KIND_F32)}
    out = {}
    for n, x in src.items():
        out[n], out[n + "_descale"] = synth.e4m3_quantize(x)
    return out


def _decoded(inp):
    return [oracle.e4m3_decode(inp[n]) * inp[n + "_descale"] for n in ("q", "k", "v")]


def check_fp8(o_gpu, lse_gpu, inp, scale, rows=None, what=""):
    """The bound of the module docstring, element by element, plus the mean-error checks."""
    qd, kd, vd = _decoded(inp)
    if rows is not None:
        qd = qd[:, :, np.asarray(rows)]
    o_ref, l_ref, P = oracle.attention(qd, kd, vd, scale, want_p=True)
    a_abs, _ = oracle.attention(qd, kd, np.abs(vd), scale)
    o = to_f64(o_gpu) if isinstance(o_gpu, torch.Tensor) else o_gpu
    l = to_f64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    if rows is not None:
        o, l = o[:, :, np.asarray(rows)], l[:, :, np.asarray(rows)]
    assert o.shape == o_ref.shape and l.shape == l_ref.shape
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), what + ": non-finite output"
    pmax = P.max(axis=-1, keepdims=True)                     # [B, H, R, 1]
    small = P < 2.0 ** -11 * pmax                            # [B, H, R, Skv]
    s_small = np.einsum("bhrj,bhjd->bhrd", small.astype(np.float64), np.abs(vd))
    bound = 2.0 ** -4 * a_abs + 2.0 ** -15 * pmax * s_small + 2.0 ** -8 * np.abs(o_ref) + 1e-6
    lbound = math.log1p(2.0 ** -4) + 2.0 ** -15 * pmax[..., 0] * small.sum(-1) + 1e-6
    err, lerr = np.abs(o - o_ref), np.abs(l - l_ref)
    worst = float(np.max(err / bound))
    msg = ("%s: O max/mean err %.3g/%.3g (worst err/bound %.3f, mean A %.3g), LSE max/mean %.3g/%.3g"
           % (what, err.max(), err.mean(), worst, a_abs.mean(), lerr.max(), lerr.mean()))
    print(msg, flush=True)
    assert np.all(err <= bound), msg
    assert np.all(lerr <= lbound), msg
    assert err.mean() <= 2.0 ** -6 * a_abs.mean(), msg
    assert lerr.mean() <= 2.0 ** -5, msg


def _run(inp, scale, out_dtype=torch.bfloat16, **kw):
    q, k, v = (_codes_to_device(inp[n]) for n in ("q", "k", "v"))
    o, l = A().chunk_fwd_fp8(q, k, v, inp["q_descale"], inp["k_descale"], inp["v_descale"], scale,
                             out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return o, l


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_fp8_all_elements(out):
    inp = _quantized(1, 3, 1000, 1500, qk=1.3)   # 1000 = 3*256 + 232 rows, 1500 = 23*64 + 28 keys
    scale = 1 / math.sqrt(128)
    o, l = _run(inp, scale, torch.bfloat16 if out == "bf16" else torch.float32)
    check_fp8(o, l, inp, scale, what="fp8 all elements out=%s" % out)


@pytest.mark.parametrize("Sq,Skv", [(1, 1), (31, 63), (33, 65), (129, 130), (257, 1), (300, 4097)])
def test_fp8_tails(Sq, Skv):
    inp = _quantized(2, 2, Sq, Skv, seed=3)
    o, l = _run(inp, 0.1)
    check_fp8(o, l, inp, 0.1, what="fp8 tails Sq=%d Skv=%d" % (Sq, Skv))


@pytest.mark.parametrize("Skv", [333, 5000])  # 5000: the balanced tail writes through the strided output
def test_fp8_strided_bshd_views(Skv):
    B, H, Sq, D = 2, 4, 200, 128
    inp = _quantized(B, H, Sq, Skv, seed=4)
    # [B, S, H, D] storage viewed as [B, H, S, D]
    q, k, v = (_codes_to_device(np.ascontiguousarray(inp[n].transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
               for n in ("q", "k", "v"))
    out = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    o, l = A().chunk_fwd_fp8(q, k, v, inp["q_descale"], inp["k_descale"], inp["v_descale"], 0.09, out=out)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    check_fp8(o, l, inp, 0.09, what="fp8 strided")


def test_fp8_uniform_values_and_descale_algebra():
    B, H, Sq, Skv, D = 1, 2, 130, 777, 128
    inp = _quantized(B, H, Sq, Skv, seed=5)
    # every value 1.0 (code 0x38) times a descale of 0.5: O is 0.5 up to the final fp32 division,
    # because the row sum adds the same rounded probabilities that P.V weighs (the E4M3
    # rounding of P cancels)
    flat = dict(inp, v=np.full_like(inp["v"], 0x38), v_descale=0.5)
    o, l = _run(flat, 0.1, torch.float32)
    assert float((o - 0.5).abs().max()) <= 2.0 ** -23
    # scaling v_descale by 2 doubles O exactly; trading a factor 2 between q_descale and the
    # scale changes nothing (the kernel's score factor is their product)
    o1, l1 = _run(inp, 0.1, torch.float32)
    o2, l2 = _run(dict(inp, v_descale=2 * inp["v_descale"]), 0.1, torch.float32)
    assert torch.equal(o2, 2 * o1) and torch.equal(l2, l1)
    o3, l3 = _run(dict(inp, q_descale=2 * inp["q_descale"]), 0.05, torch.float32)
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


def test_fp8_deterministic_workspace_reuse_and_empty():
    inp = _quantized(1, 2, 300, 900, seed=6)
    ws = torch.empty(A().fp8_workspace_size(1, 2, 300, 900, 128) + 4096, dtype=torch.uint8, device="cuda")
    o1, l1 = _run(inp, 0.1, workspace=ws)
    small = _quantized(1, 2, 300, 100, seed=7)
    _run(small, 0.1, workspace=ws)  # the same workspace, different contents in between
    o2, l2 = _run(inp, 0.1, workspace=ws)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # no keys: O = 0, LSE = -inf
    q = _codes_to_device(inp["q"])
    e = torch.empty((1, 2, 0, 128), dtype=torch.uint8, device="cuda")
    o, l = A().chunk_fwd_fp8(q, e, e, 1.0, 1.0, 1.0, 0.1)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


def test_fp8_balanced_tail():
    """Three query tiles against 79 key tiles: the work is spread over 237 workgroups of one key
    tile each, whose fp32 partials the fix-up merges (79 per row).  Within a run the lazy
    reference is the run's own, so every probability is rounded at least as finely as in one
    pass, and the merge normalises by the sum of the rounded probabilities: the bound holds."""
    inp = _quantized(1, 3, 200, 5000, seed=8)
    assert A().fp8_workspace_size(1, 3, 200, 5000, 128) > 3 * 79 * 8192  # V^T and the tail's slots
    o, l = _run(inp, 1 / math.sqrt(128))
    check_fp8(o, l, inp, 1 / math.sqrt(128), what="fp8 balanced tail")


@pytest.mark.parametrize("tail", ["ranges", "5"])
def test_fp8_persistent_dispatch(tail, monkeypatch):
    """300 query tiles (20 heads x 15) against 79 key tiles, the persistent launch forced on (the
    library's debug switch; at full size the 44,160-key shapes choose it themselves): with one
    tail run of equal units per CU bitwise equal to one workgroup per item; with the 44 tail
    tiles cut into 5 parts within the bound on sampled rows of every head."""
    B, H, Sq, Skv = 1, 20, 3600, 5000
    inp = _quantized(B, H, Sq, Skv, seed=12)
    print("fp8 persistent, tail %s" % tail, flush=True)
    monkeypatch.setenv("LSDIT_DEBUG_TAIL", tail)
    monkeypatch.setenv("LSDIT_DEBUG_PERSIST", "1")
    o, l = _run(inp, 0.1, torch.float32)
    if tail == "ranges":
        monkeypatch.setenv("LSDIT_DEBUG_PERSIST", "0")
        o_s, l_s = _run(inp, 0.1, torch.float32)
        assert torch.equal(o, o_s) and torch.equal(l, l_s)
    rows = sorted({0, 255, 256, 3583, 3584, 3599} | set(range(0, Sq, 211)))
    check_fp8(o, l, inp, 0.1, rows=rows, what="fp8 persistent tail %s" % tail)


FULL = ["image_dit", "ring_share_r0", "ulysses_share", "full_sequence"]


@pytest.mark.parametrize("name", FULL)
def test_fp8_full_size_sampled_rows(name):
    w = workloads.WORKLOADS[name]
    inp = w.make_inputs_fp8(seed=0)
    o, l = _run(inp, w.scale)
    rows = workloads.sample_rows(w.Sq, boundaries=(256, 5520), n_random=24, seed=1)
    check_fp8(o, l, inp, w.scale, rows=rows, what="fp8 %s (%d rows x %d heads)" % (name, len(rows), w.H))


@pytest.mark.parametrize("Skv", [1000, 63])
def test_fp8_rows_past_the_keys_are_not_read(Skv):
    """K and V are views of the first Skv rows of longer buffers whose rows past Skv hold the E4M3
    NaN code, and the workspace past the V^T tiles holds it too: the last, partial key tile and
    the tiles fetched past the end read zeros there, so the result stays finite and within the
    bound.  (No balanced tail at this shape: the last head's V^T tiles end where the filled
    excess of the workspace begins.)"""
    B, H, Sq, D = 1, 2, 300, 128
    inp = _quantized(B, H, Sq, Skv, seed=9)
    pad = 320
    kb = np.full((B, H, Skv + pad, D), 0x7F, np.uint8)
    vb = np.full((B, H, Skv + pad, D), 0x7F, np.uint8)
    kb[:, :, :Skv] = inp["k"]
    vb[:, :, :Skv] = inp["v"]
    q = _codes_to_device(inp["q"])
    k, v = _codes_to_device(kb)[:, :, :Skv], _codes_to_device(vb)[:, :, :Skv]
    need = A().fp8_workspace_size(B, H, Sq, Skv, D)
    assert need == B * H * -(-Skv // 64) * 8192  # V^T tiles only: no tail
    ws = torch.full((need + 65536,), 0x7F, dtype=torch.uint8, device="cuda")
    o, l = A().chunk_fwd_fp8(q, k, v, inp["q_descale"], inp["k_descale"], inp["v_descale"], 0.1, workspace=ws)
    torch.cuda.synchronize()
    check_fp8(o, l, inp, 0.1, what="fp8 NaN codes past Skv=%d" % Skv)


def test_fp8_nan_query_row_stays_in_its_row():
    """A NaN code in one query row makes that row's O and LSE NaN and leaves every other row within
    the bound: the row-sum MFMA's zero entries must not carry the NaN into the query sharing its
    column (the weights are clamped to [0, 1], NaN to 0, before the E4M3 conversion)."""
    inp = _quantized(1, 1, 64, 700, seed=10)
    q = inp["q"].copy()
    q[0, 0, 17, 5] = 0x7F
    o, l = _run(dict(inp, q=q), 0.1, torch.float32)
    assert torch.isnan(o[0, 0, 17]).all() and torch.isnan(l[0, 0, 17])
    keep = [r for r in range(64) if r != 17]
    check_fp8(o, l, inp, 0.1, rows=keep, what="fp8 NaN query row, other rows")
