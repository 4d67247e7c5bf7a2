"""Seeded synthetic inputs for MoE routing, dispatch and combine.

This module is the only code that both the HIP path's tests/benchmark and
the CPU oracle consume.  It holds the workload shapes and the draw recipes,
and none of the method's arithmetic (no selection, no softmax, no slot
assignment, no quantisation, no weighted sum).

Shapes follow the model families the pages name: Mixtral 8x7B and DeepSeek
R1 (pplx blog, Introduction), DeepSeek-V3 scale with hidden 7168 and 256
experts, top-8 (handbook, "NVSHMEM and DeepEP", simulation and fixed-slot
estimate), and the GLM MoE with hidden 6144 ("How GPUs Talk to Each Other",
section 1.1).  No dataset is involved: activations, logits and expert
outputs are drawn from seeded generators.

Recipe (per workload, seed S):
  logits  float32 [T, E]  ~ N(0, 1)               torch.Generator seeded S*16+0
  x       bf16    [T, H]  ~ N(0, 1), fp32 -> bf16  seeded S*16+1
  routing skew, applied to the logits:
    "normal": none
    "zipf"  : logits[:, e] += -1.2 * ln(rank_e), rank = a seeded random
              permutation of 1..E (seeded S*16+2)
    "hot"   : round(0.1*E) experts drawn by a seeded permutation (S*16+2)
              get logits[:, e] += 1.32
  y_pairs bf16    [T*k, H] ~ N(0, 1): the output of token t's j-th expert
              is row t*k + j (seeded S*16+3, drawn in row chunks)
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    H: int          # hidden size
    E: int          # experts
    k: int          # experts per token
    fp8: bool       # dispatch rows as E4M3 codes + per-128 fp32 scales
    C: int          # fixed slots per expert
    routing: str    # "normal" | "zipf" | "hot"
    seed: int
    desc: str = ""

    @property
    def dtype_code(self) -> int:
        return 1 if self.fp8 else 0

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 8, 2, False, 64, "normal", 1001,
                     "tiny: 64 tokens, hidden 256, 8 experts, top-2, bf16, 64 slots per expert"),
    "mixtral_prefill": Workload("mixtral_prefill", 4096, 4096, 8, 2, False, 4096, "normal", 1002,
                                "Mixtral-like prefill: 4096 tokens, hidden 4096, 8 experts, top-2, bf16"),
    "dsr1_decode": Workload("dsr1_decode", 128, 7168, 256, 8, True, 128, "normal", 1003,
                            "DeepSeek-R1-like decode: 128 tokens, hidden 7168, 256 experts, top-8, fp8 dispatch"),
    "dsr1_prefill": Workload("dsr1_prefill", 16384, 7168, 256, 8, False, 16384, "zipf", 1004,
                             "DeepSeek-R1-like prefill: 16384 tokens, hidden 7168, 256 experts, top-8, bf16, "
                             "Zipf(1.2)-skewed routing"),
    "glm_prefill": Workload("glm_prefill", 32768, 6144, 128, 8, True, 32768, "hot", 1005,
                            "GLM-style prefill: 32768 tokens, hidden 6144, 128 experts, top-8, fp8 dispatch, "
                            "10% hot experts"),
}

ORDER = ["tiny", "mixtral_prefill", "dsr1_decode", "dsr1_prefill", "glm_prefill"]

ZIPF_S = 1.2
HOT_FRACTION = 0.1
HOT_BOOST = 1.32


def _gen(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 16 + stream)
    return g


def make_logits(w: Workload) -> torch.Tensor:
    """Router logits, float32 [T, E], on the CPU."""
    logits = torch.randn(w.T, w.E, generator=_gen(w.seed, 0), dtype=torch.float32)
    if w.routing == "zipf":
        rank = torch.randperm(w.E, generator=_gen(w.seed, 2)).to(torch.float64) + 1.0
        bias = (-ZIPF_S * torch.log(rank)).to(torch.float32)
        logits += bias[None, :]
    elif w.routing == "hot":
        n_hot = int(round(HOT_FRACTION * w.E))
        hot = torch.randperm(w.E, generator=_gen(w.seed, 2))[:n_hot]
        logits[:, hot] += HOT_BOOST
    elif w.routing != "normal":
        raise ValueError(f"unknown routing {w.routing!r}")
    return logits


def hot_experts(w: Workload) -> torch.Tensor:
    """The experts that receive the boost in "hot" routing."""
    n_hot = int(round(HOT_FRACTION * w.E))
    return torch.randperm(w.E, generator=_gen(w.seed, 2))[:n_hot]


def make_x(w: Workload) -> torch.Tensor:
    """Token activations, bf16 [T, H], on the CPU."""
    return torch.randn(w.T, w.H, generator=_gen(w.seed, 1), dtype=torch.float32).to(torch.bfloat16)


def make_y_pairs(w: Workload, rows: int | None = None, chunk_rows: int = 4096) -> torch.Tensor:
    """Expert outputs, bf16 [T*k, H] (row t*k + j belongs to token t's j-th
    expert), on the CPU.  `rows` limits the draw to the first rows (the draw
    is sequential, so a prefix is the same whatever `rows` is)."""
    n = w.T * w.k if rows is None else rows
    g = _gen(w.seed, 3)
    out = torch.empty(n, w.H, dtype=torch.bfloat16)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        out[r0:r1] = torch.randn(r1 - r0, w.H, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return out


def bits(t: torch.Tensor):
    """uint16 numpy view of a bf16 tensor (bit patterns)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def from_bits(a) -> torch.Tensor:
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view("int16")).view(torch.bfloat16)
