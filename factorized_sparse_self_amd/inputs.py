"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws Gaussian tensors from a
CPU ``torch.Generator`` so that the GPU path and the fp64 oracle see identical
bytes.  The shapes are those of the workloads the Sparse Transformer pages
describe: 12,288-long byte / pixel sequences (64x64x3 images, enwik8 contexts)
and 65,536-sample audio.  The values are i.i.d. N(0, 1) stand-ins for the
projected activations; the datasets themselves are not used.

Recipe (identical on every machine): ``torch.Generator().manual_seed(seed)``,
draws in the order q, k, v, dO, each ``randn(B, H, T, D)`` in fp32, multiplied
by ``scale`` and then rounded to the compute dtype (round-to-nearest-even for
bf16 and fp16).  The oracle receives these stored values widened exactly to fp64.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

STRIDED, FIXED, FIXED_R1, DENSE, STRIDED_UNION, FIXED_UNION = range(6)
PATTERN_NAMES = {STRIDED: "strided", FIXED: "fixed", FIXED_R1: "fixed_r1", DENSE: "dense",
                 STRIDED_UNION: "strided_union", FIXED_UNION: "fixed_union"}


def summary_offsets(l: int, c) -> tuple:
    """A workload's summary offsets: the last c of each block, or the given ones."""
    return tuple(range(l - c, l)) if isinstance(c, int) else tuple(sorted(c))


@dataclass(frozen=True)
class Workload:
    """One attention problem: pattern, shapes, dtype and the passes it runs."""

    name: str
    pattern: int
    B: int
    H: int
    T: int
    D: int
    l: int
    c: object  # summary count (its last c offsets), or the summary offsets (a tuple)
    dtype: str  # "bf16", "f16" or "f32"
    backward: bool
    seed: int
    scale: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[self.dtype]


# The five workloads of the hot path.  Seeds are 1000 + position.
WORKLOADS = [
    Workload("strided_T256_f32_fwd", STRIDED, 1, 2, 256, 32, 16, 0, "f32", False, 1000,
             note="head0 = previous 16 positions, head1 = every 16th earlier position"),
    Workload("fixed_T1024_bf16_fwd", FIXED, 2, 4, 1024, 64, 32, 4, "bf16", False, 1001, 0.5,
             note="c = 4 summary positions at the end of each 32-block, alternating heads"),
    Workload("strided_T12288_bf16_fwd", STRIDED, 1, 16, 12288, 64, 128, 0, "bf16", False, 1002,
             note="64x64x3 pixel-order sequence, 8 local + 8 strided heads"),
    Workload("fixed_T12288_bf16_fwdbwd", FIXED, 4, 8, 12288, 64, 128, 8, "bf16", True, 1003,
             note="enwik8-length context, c = 8, forward + recompute backward"),
    Workload("strided_T65536_bf16_fwdbwd", STRIDED, 1, 8, 65536, 64, 256, 0, "bf16", True, 1004,
             note="audio-length sequence, 4 local + 4 strided heads"),
]
# Follow-up workloads: full causal attention at the fixed workload's shape (the
# comparator of the pages' fixed-vs-full training-step timing), the summary
# variant whose summary keys include the query's own block up to t, and a
# million-length strided sequence, and merged heads (every head attends both
# sets) at the 12,288-long shapes.
EXTRA_WORKLOADS = [
    Workload("dense_T12288_bf16_fwdbwd", DENSE, 4, 8, 12288, 64, 128, 0, "bf16", True, 1005,
             note="full causal attention at the fixed workload's shape"),
    Workload("fixed_r1_T12288_bf16_fwdbwd", FIXED_R1, 4, 8, 12288, 64, 128, 8, "bf16", True, 1006,
             note="summary keys of earlier blocks and of the own block up to t"),
    Workload("strided_T1048576_bf16_fwdbwd", STRIDED, 1, 2, 1 << 20, 64, 1024, 0, "bf16", True, 1007,
             note="million-length sequence, one local and one strided head"),
    Workload("fixed_union_T12288_bf16_fwdbwd", FIXED_UNION, 4, 8, 12288, 64, 128, 8, "bf16", True, 1008,
             note="merged heads: own block plus earlier summary keys in every head"),
    Workload("strided_union_T12288_bf16_fwdbwd", STRIDED_UNION, 1, 16, 12288, 64, 128, 0, "bf16", True, 1009,
             note="merged heads: window plus strided keys in every head"),
    Workload("fixed_T12288_f16_fwdbwd", FIXED, 4, 8, 12288, 64, 128, 8, "f16", True, 1010,
             note="the fixed workload with fp16 (IEEE binary16) inputs"),
    Workload("fixed_spread_T12288_bf16_fwdbwd", FIXED, 4, 8, 12288, 64, 128, tuple(range(0, 128, 16)), "bf16",
             True, 1011, note="the fixed workload with 8 summary offsets spread over each block"),
    Workload("fixed_D128_T12288_bf16_fwdbwd", FIXED, 4, 8, 12288, 128, 128, 8, "bf16", True, 1012,
             note="the fixed workload with head dimension 128"),
    Workload("fixed_T12287_bf16_fwdbwd", FIXED, 4, 8, 12287, 64, 128, 8, "bf16", True, 1013,
             note="the fixed workload one position short: T a multiple of neither l nor the 64-row block"),
]
WORKLOAD_BY_NAME = {w.name: w for w in WORKLOADS + EXTRA_WORKLOADS}


def draw(B: int, H: int, T: int, D: int, *, dtype: torch.dtype, seed: int,
         scale: float = 1.0, n: int = 3) -> list[torch.Tensor]:
    """Return ``n`` CPU tensors [B, H, T, D] (q, k, v[, dO]) drawn from ``seed``."""
    g = torch.Generator().manual_seed(int(seed))
    out = []
    for _ in range(n):
        x = torch.randn(B, H, T, D, generator=g, dtype=torch.float32)
        if scale != 1.0:
            x = x * scale
        out.append(x.to(dtype).contiguous())
    return out


def draw_workload(w: Workload, *, n: int | None = None) -> list[torch.Tensor]:
    """q, k, v (and dO when the workload has a backward) for one workload, on the CPU."""
    if n is None:
        n = 4 if w.backward else 3
    return draw(w.B, w.H, w.T, w.D, dtype=w.torch_dtype, seed=w.seed, scale=w.scale, n=n)
