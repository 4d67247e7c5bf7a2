"""Helpers for the GPU parity tests: device checks, bf16 ulp distance, and
running the HIP path (through the C ABI binding) and the CPU oracle on the
same seeded inputs.  No expected value here comes from the HIP path."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as W

# Router weights: the GPU computes the softmax in fp32 (expf, per-lane sums
# then a butterfly), the oracle in fp64 rounded once.  Bound on the fp32
# path's relative error: the logit difference rounds by <= 2^-24 |d| with
# |d| <= 16 here (<= 2^-20 relative in exp), expf itself ~2^-23, the sum of
# <= 1024 terms through 16 sequential adds and a 6-level butterfly
# accumulates <= 22 * 2^-24, the divide 2^-24: about 2^-18.5 in total.
# The tolerance takes 2^-17.
W_RTOL = 2.0 ** -17


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device (torch.cuda.is_available() is False)")
    import combine_moe_route_amd as m
    m.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_ordered(bits_u16: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers whose difference counts ulps
    (sign-magnitude -> two's complement order; +0 and -0 coincide)."""
    b = bits_u16.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(bf16_ordered(a_bits) - bf16_ordered(b_bits))


def dev_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> host uint16 bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_bf16(bits_u16: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(device).view(torch.bfloat16)


class OracleRun:
    """Oracle results for a workload (cached per process)."""
    _cache: dict = {}

    def __init__(self, w: W.Workload):
        self.w = w
        self.logits = W.make_logits(w).numpy()
        self.x = W.bits(W.make_x(w))
        self.idx, self.wt = oracle.route_topk(self.logits, w.k)
        self.counts, self.token_slot, self.recv_src = oracle.assign_slots(self.idx, w.E, w.C)
        self._y = None

    @classmethod
    def get(cls, w: W.Workload) -> "OracleRun":
        if w not in cls._cache:
            cls._cache.clear()       # keep one workload's arrays alive at a time
            cls._cache[w] = OracleRun(w)
        return cls._cache[w]

    @property
    def y_pairs(self) -> np.ndarray:
        if self._y is None:
            self._y = W.bits(W.make_y_pairs(self.w))
        return self._y


def place_rows(w: W.Workload, y_pairs_bits: np.ndarray, token_slot: np.ndarray, device) -> torch.Tensor:
    """Expert-output buffer [E, C, H] on the device with row t*k+j of y_pairs
    at the slot the oracle assigned to (t, j) (test plumbing, torch ops)."""
    y = torch.empty(w.E, w.C, w.H, dtype=torch.bfloat16, device=device)
    flat = token_slot.reshape(-1)
    keep = np.nonzero(flat >= 0)[0]
    rows = to_dev_bf16(y_pairs_bits[keep], device)
    dst = torch.from_numpy(flat[keep].astype(np.int64)).to(device)
    y.view(-1, w.H).index_copy_(0, dst, rows)
    return y
