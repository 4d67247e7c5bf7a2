"""Seeded random shapes through both fused entry points (moe_route_dispatch
with fixed slots, moe_route_dispatch_packed) and combine, against the
oracle: E from 1 to 300, k up to min(E, 16), T from 1 to 3000 (single
chunk, router-word and multi-chunk paths), ragged H, bf16 and fp8 rows,
capacity below and above the largest count, ties in the logits.  Ids,
counts, offsets, slots, sources and row contents bit for bit; weights within
the router tolerance; combine of identity experts (each slot's output is its
dispatched bf16 row) within one bf16 ulp."""
import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
import oracle
import workloads as W
from gpu_common import W_RTOL, bf16_ulp_distance, dev_bits, require_gpu, say, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _case(seed):
    rng = np.random.default_rng(70_000 + seed)
    E = int(rng.choice([1, 2, 3, 5, 8] + [int(rng.integers(9, 301)) for _ in range(4)]))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.choice([int(rng.integers(1, 257)), int(rng.integers(257, 3001)), int(rng.integers(257, 3001))]))
    fp8 = bool(rng.integers(0, 2))
    H = 128 * int(rng.integers(1, 9)) if fp8 else 8 * int(rng.integers(1, 101))
    if rng.random() < 0.3:
        logits = rng.integers(-2, 3, (T, E)).astype(np.float32)          # ties
    else:
        logits = rng.standard_normal((T, E)).astype(np.float32)
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    C = int(rng.integers(max(1, T * k // max(E, 1) // 2), T + 1))
    return E, k, T, H, fp8, C, logits, x


def _rows_match(got_rows, x_bits, src, fp8, H):
    if fp8:
        codes, scales = oracle.quantize_rows_fp8(x_bits)
        return codes[src], scales[src]
    return x_bits[src], None


@pytest.mark.parametrize("seed", range(200))
def test_random_fused_paths(dev, seed):
    E, k, T, H, fp8, C, logits, x = _case(seed)
    say(f"[random] seed={seed} T={T} E={E} k={k} H={H} C={C} fp8={fp8}")
    lg = torch.from_numpy(logits).to(dev)
    xd = to_dev_bf16(x, dev)
    idx_o, w_o = oracle.route_topk(logits, k)

    # fixed slots
    idx, wt, b = moe.moe_route_dispatch(lg, xd, k, C, fp8=fp8)
    counts_o, slot_o, src_o = oracle.assign_slots(idx_o, E, C)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    wt_h = wt.cpu().numpy()
    np.testing.assert_allclose(wt_h, w_o, rtol=W_RTOL, atol=0)
    np.testing.assert_array_equal(b.expert_counts.cpu().numpy(), counts_o)
    np.testing.assert_array_equal(b.token_slot.cpu().numpy(), slot_o)
    filled = src_o >= 0
    np.testing.assert_array_equal(b.recv_src.cpu().numpy().reshape(-1)[filled], src_o[filled])
    rows_o, sc_o = _rows_match(None, x, src_o[filled], fp8, H)
    if fp8:
        np.testing.assert_array_equal(b.recv_x.view(E * C, H).cpu().numpy()[filled], rows_o)
        np.testing.assert_array_equal(b.recv_scales.view(E * C, H // 128).cpu().numpy()[filled], sc_o)
    else:
        np.testing.assert_array_equal(dev_bits(b.recv_x.view(E * C, H))[filled], rows_o)
        # identity experts: combine reads back the dispatched rows
        out = moe.moe_combine(b.recv_x, b.token_slot, wt)
        y_pairs = np.where((slot_o.reshape(-1) >= 0)[:, None], np.repeat(x, k, axis=0), 0).astype(np.uint16)
        ref = oracle.combine(y_pairs, slot_o, wt_h)
        assert bf16_ulp_distance(dev_bits(out), ref).max(initial=0) <= 1

    # packed layout
    idx2, wt2, p = moe.moe_route_dispatch_packed(lg, xd, k, fp8=fp8)
    offs_o, pslot_o, psrc_o = oracle.assign_packed(idx_o, E)
    assert torch.equal(idx2, idx) and torch.equal(wt2.view(torch.int32), wt.view(torch.int32))
    np.testing.assert_array_equal(p.expert_offsets.cpu().numpy(), offs_o)
    np.testing.assert_array_equal(p.token_slot.cpu().numpy(), pslot_o)
    np.testing.assert_array_equal(p.recv_src.cpu().numpy().reshape(-1)[:T * k], psrc_o)
    rows_o, sc_o = _rows_match(None, x, psrc_o, fp8, H)
    if fp8:
        np.testing.assert_array_equal(p.recv_x.cpu().numpy(), rows_o)
        np.testing.assert_array_equal(p.recv_scales.cpu().numpy(), sc_o)
    else:
        np.testing.assert_array_equal(dev_bits(p.recv_x), rows_o)
        out = moe.moe_combine(p.recv_x, p.token_slot, wt2)
        ref = oracle.combine(np.repeat(x, k, axis=0), pslot_o, wt_h)
        assert bf16_ulp_distance(dev_bits(out), ref).max(initial=0) <= 1
