"""Exhaustive parity of the fp8 dispatch encoding (handbook "NVSHMEM and
DeepEP", "High-throughput mode": FP8 with one scale per 128 elements).

Every 128-element scale block is determined by its largest magnitude a and
its values x with |x| <= a.  These rows enumerate that whole domain for bf16
activations: for every positive finite bf16 a, a block holds a in element 0
and 127 further values drawn, in order, from every bf16 x with |x| <= a (both
signs, both zeros), so ~1.07e9 (a, x) pairs in ~8.4e6 rows.  moe_dispatch
(E = 1, k = 1) packs each row into its slot; every code and scale must equal
the CPU oracle's, which divides and rounds by the E4M3 definition.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
import oracle
from gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu

AMAX_LAST = 0x7F7F      # largest finite positive bf16
N_CHUNKS = 8


def _rows_for(a_lo: int, a_hi: int) -> np.ndarray:
    """Rows for amax bit patterns a_lo .. a_hi - 1."""
    blocks = []
    for a in range(a_lo, a_hi):
        mags = np.arange(a + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | np.uint16(0x8000)])
        n_rows = -(-vals.size // 127)
        pad = np.zeros(n_rows * 127, np.uint16)
        pad[: vals.size] = vals
        rows = np.empty((n_rows, 128), np.uint16)
        rows[:, 0] = a
        rows[:, 1:] = pad.reshape(n_rows, 127)
        blocks.append(rows)
    return np.concatenate(blocks)


def _oracle_rows(x: np.ndarray):
    workers = max(1, min(16, os.cpu_count() or 1))
    parts = np.array_split(np.arange(x.shape[0]), workers)
    with cf.ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda p: oracle.quantize_rows_fp8(x[p[0]:p[-1] + 1]) if p.size else None, parts))
    res = [r for r in res if r is not None]
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def test_fp8_dispatch_matches_oracle_on_whole_domain():
    dev = require_gpu()
    # split amax values so chunks hold similar numbers of pairs (~a^2 growth)
    edges = [int(round(AMAX_LAST * (i / N_CHUNKS) ** 0.5)) + 1 for i in range(N_CHUNKS + 1)]
    edges[0], edges[-1] = 1, AMAX_LAST + 1
    total = 0
    for lo, hi in zip(edges[:-1], edges[1:]):
        x = _rows_for(lo, hi)
        T = x.shape[0]
        say(f"[fp8 exhaustive] amax 0x{lo:04x}..0x{hi - 1:04x}: {T} rows")
        codes_o, scales_o = _oracle_rows(x)
        xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        idx = torch.zeros(T, 1, dtype=torch.int32, device=dev)
        bufs = moe.moe_dispatch(xd, idx, 1, T, fp8=True)
        codes_g = bufs.recv_x.view(T, 128).cpu().numpy()
        scales_g = bufs.recv_scales.view(T).cpu().numpy()
        bad = np.nonzero((codes_g != codes_o).any(axis=1))[0]
        if bad.size:
            r = bad[0]
            col = np.nonzero(codes_g[r] != codes_o[r])[0][0]
            raise AssertionError(f"{bad.size} rows differ; first: amax 0x{x[r, 0]:04x} x 0x{x[r, col]:04x} "
                                 f"gpu 0x{codes_g[r, col]:02x} oracle 0x{codes_o[r, col]:02x}")
        np.testing.assert_array_equal(scales_g, scales_o.reshape(-1))
        assert (bufs.token_slot.cpu().numpy().reshape(-1) == np.arange(T)).all()
        total += T * 127
        del xd, idx, bufs
        torch.cuda.empty_cache()
    assert total >= 1_065_402_238
