"""The shard call captured in a HIP graph (through torch.cuda.graph) and replayed.

A persistent launch clears its work-queue counters with a kernel, not a memset, so that it can
be captured; the allocation-free entry point is meant for callers under capture.  Each graph is
replayed several times, with the program's own eager work (overwriting the outputs and the
workspace) and synchronisations between replays, and every replay must give bitwise the eager
result.
"""
import pytest
import torch

import synth
from parity_util import to_device

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
    return tuple(to_device(synth.normal_rows(seed, i, B, H, S, D, kind=synth.KIND_BF16))
                 for i, S in enumerate((Sq, Skv, Skv)))


def _replays(call, out, lse, scratch, n=3):
    """Eager result, then capture `call` and replay it n times, scribbling over the outputs and
    `scratch` eagerly before each replay; returns (eager, [replays])."""
    call()
    torch.cuda.synchronize()
    o_ref, l_ref = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture's side stream, as torch advises
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    got = []
    for i in range(n):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        if scratch is not None:
            scratch.fill_(0xA5 + i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got.append((out.clone(), lse.clone()))
    return (o_ref, l_ref), got


@pytest.mark.parametrize("mode", ["fused", "online"])
def test_persistent_shard_call_replays_bitwise(mode, monkeypatch):
    """300 query tiles against 5000 keys in two chunks, the launch forced persistent with the
    tail in 5 parts: the queue-clearing kernel, the forward kernel(s) and the fix-up captured
    and replayed."""
    monkeypatch.setenv("LSDIT_DEBUG_PERSIST", "1")
    monkeypatch.setenv("LSDIT_DEBUG_TAIL", "5")
    B, H, Sq, Skv, D = 1, 20, 3600, 5000, 128
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=51)
    lens, order = (2000, 3000), (1, 0)
    ws = torch.empty(A().shard_workspace_size(B, H, Sq, D, 2, mode), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    print("graph replay, persistent, %s" % mode, flush=True)
    call = lambda: A().shard_fwd(q, k, v, lens, order, mode=mode, out=out, lse=lse, workspace=ws)
    (o_ref, l_ref), got = _replays(call, out, lse, ws)
    assert torch.isfinite(o_ref.float()).all()
    for o, l in got:
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_noalloc_call_replays_bitwise():
    """The allocation-free entry point (static scratch, balanced tail) captured and replayed."""
    B, H, Sq, Skv, D = 1, 3, 600, 9000, 128
    q, k, v = _inputs(B, H, Sq, Skv, D, seed=52)
    lens, order = (3000, 6000), (1, 0)
    out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    print("graph replay, noalloc", flush=True)
    call = lambda: A().shard_fwd_noalloc(q, k, v, lens, order, out, lse)
    (o_ref, l_ref), got = _replays(call, out, lse, None)
    assert torch.isfinite(o_ref.float()).all()
    for o, l in got:
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
