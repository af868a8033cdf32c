"""The measurement script's own checks, on the CPU: the every-row comparison (`--full-check`) must
fail when an output element is off by more than the gate, and a committed rocprofv3 summary is
used only for the kernel source it was taken of.

The full check runs here on a small stand-in for the ring share (one head, 300 query rows against
all 44,160 keys in the ring's eight chunks) with a stub in place of the library: the stub returns
the oracle's own result rounded to bf16, so every row passes, and then the same with one element
moved past the gate, which must fail.
"""
import dataclasses
import importlib.util
import os
import types

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


class _StubLibrary:
    """shard_fwd returning the oracle's attention of the host inputs, as bf16 O and fp32 LSE,
    with `bump` added to one output element (row 7, head 0, d 3)."""

    def __init__(self, host, scale, bump=0.0):
        o, l = oracle.attention(host["q"], host["k"], host["v"], scale)
        o = o.copy()
        o[0, 0, 7, 3] += bump
        self.o = torch.from_numpy(synth.f32_to_bf16_bits(o.astype(np.float32)).view(np.int16)).view(torch.bfloat16)
        self.l = torch.from_numpy(l.astype(np.float32))
        self.calls = []

    def shard_fwd(self, q, k, v, lens, order, mode):
        self.calls.append((tuple(lens), None if order is None else tuple(order), mode))
        return self.o, self.l


@pytest.fixture(scope="module")
def small_ring_share():
    w = dataclasses.replace(workloads.RING_SHARE, H=1, Sq=300)
    return w, w.make_inputs()


def _run(bench, w, host, lib):
    fake_torch = types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda: None), int16=torch.int16)
    return bench.full_check(lib, fake_torch, w, host, None, None, None,
                            runs=((None, "fused"), (None, "online")), block_rows=128)


def test_full_check_passes_the_oracles_own_result(bench, small_ring_share):
    w, host = small_ring_share
    lib = _StubLibrary(host, w.scale)
    out = _run(bench, w, host, lib)
    assert out["rows"] == w.H * w.Sq and out["workload"] == w.name
    assert set(out["plans"]) == {"ring/fused", "ring/online"}
    for r in out["plans"].values():
        assert r["pass"] and r["nonfinite"] == 0
        assert r["o_max_abs"] <= 2.0 ** -8 and r["lse_max_abs"] <= 1e-5  # the bf16 rounding only
    # the workload's own plan (eight chunks in ring order), once per schedule
    assert [c[2] for c in lib.calls] == ["fused", "online"]
    assert all(c[0] == w.plan().lens and c[1] == w.plan().order for c in lib.calls)


def test_full_check_fails_an_element_past_the_gate(bench, small_ring_share):
    w, host = small_ring_share
    out = _run(bench, w, host, _StubLibrary(host, w.scale, bump=0.03))
    for r in out["plans"].values():
        assert not r["pass"] and 0.029 <= r["o_max_abs"] <= 0.031


def test_profile_figures_only_for_the_source_they_were_taken_of(bench, tmp_path):
    """A summary's machine-readable figures are read when its recorded hash is that of the kernel
    source as it is now, and ignored otherwise (so that a kernel change leaves the bench line's
    traffic null until the counters are taken again)."""
    body = ("plan: chunks1\nkernel_source_sha256_16: %s\ntrace_mean_kernel_us: 12345.6\n"
            "effective_clock_mhz: 1600.0\nmfma_busy: 0.77\nhbm_bytes_per_launch: 3.2e+09\n")
    current = tmp_path / "current.txt"
    current.write_text(body % bench.kernel_source_hash())
    got = bench.read_profile(str(current))
    assert got is not None and got["plan"] == "chunks1"
    assert got["trace_mean_kernel_us"] == 12345.6 and got["hbm_bytes_per_launch"] == 3.2e9
    stale = tmp_path / "stale.txt"
    stale.write_text(body % "0000000000000000")
    assert bench.read_profile(str(stale)) is None
    # comments and whitespace do not change the hash; code does
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }  // one\n")
    h = bench.kernel_source_hash([str(src)])
    src.write_text("int f() {\n  return 1;  /* two */\n}\n")
    assert bench.kernel_source_hash([str(src)]) == h
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash([str(src)]) != h
