"""The five attention workloads, as shapes plus input recipes (no attention arithmetic).

All tensors are [B, H, S, D] with d contiguous.  Values are N(0, 1) draws from
the seeded Philox stream (tensor ids Q=0, K=1, V=2), scaled in fp64 before
rounding.  The long shapes stand in for the 44,160-token Cosmos 3 Nano video
sequence and a joint image+text FLUX-style latent (NVIDIA Technical Blog,
"Scaling AI Inference Across Multiple GPUs Using NVIDIA TensorRT with
Multi-Device Inference Support", sections "Video generation with NVIDIA
Cosmos 3" and "Image generation with Flux.1"); no trained weights or prompts
are involved.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

import synth

SEQ_VIDEO = 44160


def even_chunks(total: int, n: int) -> List[int]:
    base, rem = divmod(total, n)
    return [base + (1 if i < rem else 0) for i in range(n)]


def ragged_chunks(total: int, first: int, step: int) -> List[int]:
    """first, first+step, ... while the running sum stays <= total; a final chunk takes the rest."""
    out, acc, c = [], 0, first
    while acc + c <= total:
        out.append(c)
        acc += c
        c += step
    if acc < total:
        out.append(total - acc)
    return out


def ring_order(rank: int, n: int) -> List[int]:
    """Receive-from-left ring: at step t rank r holds the chunk of rank (r - t) mod n."""
    return [(rank - t) % n for t in range(n)]


@dataclasses.dataclass(frozen=True)
class ChunkPlan:
    lens: Tuple[int, ...]
    order: Optional[Tuple[int, ...]] = None  # None = 0..n-1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Skv: int
    D: int
    dtype: str                     # "fp32" or "bf16"
    plans: Dict[str, ChunkPlan]
    default_plan: str
    s_full: int = 0                # Q is rows [q_row_lo, q_row_lo + Sq) of an s_full-row tensor
    q_row_lo: int = 0
    qk_factor: float = 1.0         # applied to Q and K in fp64 before rounding
    outlier_count: int = 0         # K rows (same positions for every head) scaled by outlier_factor
    outlier_factor: float = 8.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        return 4.0 * self.B * self.H * self.Sq * self.Skv * self.D

    def plan(self, name: Optional[str] = None) -> ChunkPlan:
        return self.plans[name or self.default_plan]

    def outlier_positions(self, seed: int = 0) -> np.ndarray:
        if self.outlier_count == 0:
            return np.zeros(0, dtype=np.int64)
        return synth.outlier_rows(seed, self.Skv, self.outlier_count)

    def make_inputs(self, seed: int = 0) -> Dict[str, np.ndarray]:
        """Host buffers q, k, v: float32 arrays (fp32) or uint16 bf16 bit patterns (bf16)."""
        kind = synth.KIND_F32 if self.dtype == "fp32" else synth.KIND_BF16
        s_full = self.s_full or self.Sq
        q = synth.normal_rows(seed, synth.TID_Q, self.B, self.H, s_full, self.D,
                              self.q_row_lo, self.q_row_lo + self.Sq, self.qk_factor, None, kind)
        row_factor = None
        if self.outlier_count:
            row_factor = np.ones(self.Skv)
            row_factor[self.outlier_positions(seed)] = self.outlier_factor
        k = synth.normal_rows(seed, synth.TID_K, self.B, self.H, self.Skv, self.D, 0, self.Skv,
                              self.qk_factor, row_factor, kind)
        v = synth.normal_rows(seed, synth.TID_V, self.B, self.H, self.Skv, self.D, 0, self.Skv, 1.0, None, kind)
        return {"q": q, "k": k, "v": v}


    def make_inputs_fp8(self, seed: int = 0) -> Dict[str, object]:
        """E4M3 codes (uint8, [B, H, S, D]) of the same draws as make_inputs, each tensor
        quantized per tensor from its fp32 values; descales in "q_descale" etc."""
        s_full = self.s_full or self.Sq
        src = {
            "q": synth.normal_rows(seed, synth.TID_Q, self.B, self.H, s_full, self.D, self.q_row_lo,
                                   self.q_row_lo + self.Sq, self.qk_factor, None, synth.KIND_F32),
        }
        row_factor = None
        if self.outlier_count:
            row_factor = np.ones(self.Skv)
            row_factor[self.outlier_positions(seed)] = self.outlier_factor
        src["k"] = synth.normal_rows(seed, synth.TID_K, self.B, self.H, self.Skv, self.D, 0, self.Skv,
                                     self.qk_factor, row_factor, synth.KIND_F32)
        src["v"] = synth.normal_rows(seed, synth.TID_V, self.B, self.H, self.Skv, self.D, 0, self.Skv, 1.0, None,
                                     synth.KIND_F32)
        out: Dict[str, object] = {}
        for name, x in src.items():
            codes, descale = synth.e4m3_quantize(x)
            out[name] = codes
            out[name + "_descale"] = descale
        return out

def _even_plans(total: int, counts) -> Dict[str, ChunkPlan]:
    return {"chunks%d" % n: ChunkPlan(tuple(even_chunks(total, n))) for n in counts}


TINY = Workload("tiny", 1, 2, 256, 256, 64, "fp32",
                plans={"chunks4": ChunkPlan((64, 64, 64, 64)), "chunks1": ChunkPlan((256,))},
                default_plan="chunks4")

IMAGE_DIT = Workload("image_dit", 1, 24, 4608, 4608, 128, "bf16",
                     plans={"chunks1": ChunkPlan((4608,))}, default_plan="chunks1")


def ring_share(rank: int = 0, n_ranks: int = 8) -> Workload:
    sq = SEQ_VIDEO // n_ranks
    plans = {"ring": ChunkPlan(tuple(even_chunks(SEQ_VIDEO, n_ranks)), tuple(ring_order(rank, n_ranks)))}
    return Workload("ring_share_r%d" % rank, 1, 16, sq, SEQ_VIDEO, 128, "bf16", plans=plans,
                    default_plan="ring", s_full=SEQ_VIDEO, q_row_lo=rank * sq)


RING_SHARE = ring_share(0)

ULYSSES_SHARE = Workload("ulysses_share", 1, 4, SEQ_VIDEO, SEQ_VIDEO, 128, "bf16",
                         plans={"chunks1": ChunkPlan((SEQ_VIDEO,))}, default_plan="chunks1",
                         qk_factor=1.5)

_full_plans = _even_plans(SEQ_VIDEO, (1, 2, 4, 8))
_full_plans["ragged"] = ChunkPlan(tuple(ragged_chunks(SEQ_VIDEO, 5000, 1000)))
_full_plans["ring8"] = ChunkPlan(tuple(even_chunks(SEQ_VIDEO, 8)), tuple(ring_order(0, 8)))
FULL_SEQUENCE = Workload("full_sequence", 1, 16, SEQ_VIDEO, SEQ_VIDEO, 128, "bf16", plans=_full_plans,
                         default_plan="chunks1", outlier_count=SEQ_VIDEO // 100)

WORKLOADS = {w.name: w for w in (TINY, IMAGE_DIT, RING_SHARE, ULYSSES_SHARE, FULL_SEQUENCE)}


def sample_rows(Sq: int, boundaries=(), n_random: int = 0, seed: int = 0) -> np.ndarray:
    """Query rows to check one by one: edges of 64/128/256-row tiles near both ends,
    every given boundary +-1, the last row, and n_random seeded rows."""
    rows = {0, 1, Sq - 1, Sq - 2}
    for t in (64, 128, 256):
        for base in (t, Sq - Sq % t if Sq % t else Sq - t):
            for d in (-1, 0, 1):
                rows.add(base + d)
    for b in boundaries:
        for d in (-1, 0, 1):
            rows.add(b + d)
    if n_random:
        w = synth.raw_u32(seed, 7, 0, n_random)
        rows.update(int(x) % Sq for x in w)
    return np.array(sorted(r for r in rows if 0 <= r < Sq), dtype=np.int64)
