"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
the five seeded workloads, at their full sizes and in the launch
configuration the benchmark uses.

  route:    expert ids bit-exact, weights within W_RTOL of the oracle
  dispatch: counts, token_slot, recv_src and every filled recv_x row (bf16
            bits, or E4M3 codes plus fp32 scales) bit-exact
  combine:  <= 1 bf16 ulp from the oracle (fp32 FMA in top-k order; the
            same operation order on both sides, so 0 ulp is expected)
  pipeline: route -> dispatch -> combine on the GPU end to end
"""
import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
import oracle
import workloads as W
from gpu_common import (W_RTOL, OracleRun, bf16_ulp_distance, dev_bits, place_rows, require_gpu, say,
                        to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", W.ORDER)
def test_route_parity(dev, name):
    w = W.WORKLOADS[name]
    say(f"[route] {name} T={w.T} E={w.E} k={w.k}")
    o = OracleRun.get(w)
    idx, wt = moe.moe_route_topk(torch.from_numpy(o.logits).to(dev), w.k)
    idx, wt = idx.cpu().numpy(), wt.cpu().numpy()
    np.testing.assert_array_equal(idx, o.idx)
    np.testing.assert_allclose(wt, o.wt, rtol=W_RTOL, atol=0)


def _filled_rows(bufs, w, slot_of_row, dev):
    sel = torch.from_numpy(slot_of_row.astype(np.int64)).to(dev)
    rows = bufs.recv_x.view(w.E * w.C, w.H).index_select(0, sel)
    if w.fp8:
        sc = bufs.recv_scales.view(w.E * w.C, w.H // 128).index_select(0, sel).cpu().numpy()
        return rows.cpu().numpy(), sc
    return dev_bits(rows), None


@pytest.mark.parametrize("name", W.ORDER)
def test_dispatch_parity(dev, name):
    w = W.WORKLOADS[name]
    say(f"[dispatch] {name} T={w.T} H={w.H} E={w.E} k={w.k} C={w.C} fp8={w.fp8}")
    o = OracleRun.get(w)
    x = to_dev_bf16(o.x, dev)
    idx = torch.from_numpy(o.idx).to(dev)
    bufs = moe.moe_dispatch(x, idx, w.E, w.C, fp8=w.fp8)
    counts = bufs.expert_counts.cpu().numpy()
    token_slot = bufs.token_slot.cpu().numpy()
    recv_src = bufs.recv_src.cpu().numpy().reshape(-1)
    np.testing.assert_array_equal(counts, o.counts)
    np.testing.assert_array_equal(token_slot, o.token_slot)
    filled = o.recv_src >= 0
    np.testing.assert_array_equal(recv_src[filled], o.recv_src[filled])
    slot_of_row = np.nonzero(filled)[0]
    rows, scales = _filled_rows(bufs, w, slot_of_row, dev)
    src = o.recv_src[slot_of_row]
    if w.fp8:
        codes_tok, scales_tok = oracle.quantize_rows_fp8(o.x)
        np.testing.assert_array_equal(scales, scales_tok[src])
        np.testing.assert_array_equal(rows, codes_tok[src])
    else:
        np.testing.assert_array_equal(rows, o.x[src])
    del bufs, x, idx
    _free()


def _combine_check(out_bits, want_bits, label):
    d = bf16_ulp_distance(out_bits, want_bits)
    n_off = int((d != 0).sum())
    say(f"  {label}: max ulp {int(d.max()) if d.size else 0}, elements not bit-identical {n_off} of {d.size}")
    assert d.max(initial=0) <= 1


@pytest.mark.parametrize("name", W.ORDER)
def test_combine_parity(dev, name):
    w = W.WORKLOADS[name]
    say(f"[combine] {name} T={w.T} H={w.H} E={w.E} k={w.k} C={w.C}")
    o = OracleRun.get(w)
    y_pairs = o.y_pairs
    want = oracle.combine(y_pairs, o.token_slot, o.wt)
    y = place_rows(w, y_pairs, o.token_slot, dev)
    out = moe.moe_combine(y, torch.from_numpy(o.token_slot).to(dev), torch.from_numpy(o.wt).to(dev))
    _combine_check(dev_bits(out), want, name)
    del y, out
    _free()


@pytest.mark.parametrize("name", W.ORDER)
def test_pipeline_end_to_end(dev, name):
    """The benchmark's step: route, dispatch, combine on one stream; the
    expert outputs are the dispatched rows themselves for bf16 workloads
    (identity experts) and the seeded outputs for fp8 ones."""
    w = W.WORKLOADS[name]
    say(f"[pipeline] {name}")
    o = OracleRun.get(w)
    logits = torch.from_numpy(o.logits).to(dev)
    x = to_dev_bf16(o.x, dev)
    idx, wt = moe.moe_route_topk(logits, w.k)
    bufs = moe.moe_dispatch(x, idx, w.E, w.C, fp8=w.fp8)
    if w.fp8:
        y_pairs = o.y_pairs
        y = place_rows(w, y_pairs, o.token_slot, dev)
    else:
        y_pairs = np.repeat(o.x, w.k, axis=0)      # identity experts
        y = bufs.recv_x
    out = moe.moe_combine(y, bufs.token_slot, wt)
    np.testing.assert_array_equal(idx.cpu().numpy(), o.idx)
    np.testing.assert_array_equal(bufs.token_slot.cpu().numpy(), o.token_slot)
    wt_gpu = wt.cpu().numpy()
    # oracle combine with the oracle's weights; the GPU used its own fp32
    # weights, so allow their tolerance on top of one bf16 ulp
    want, acc = oracle.combine(y_pairs, o.token_slot, o.wt, want_acc=True)
    got = dev_bits(out)
    d = bf16_ulp_distance(got, want)
    t_i, h_i = np.nonzero(d > 1)
    n_bad = 0
    if t_i.size:
        yv = (y_pairs.reshape(w.T, w.k, w.H)[t_i, :, h_i].astype(np.uint32) << 16).view(np.float32)
        mag = (np.abs(o.wt[t_i]).astype(np.float64) * np.abs(yv).astype(np.float64)).sum(axis=1)
        gotf = (got[t_i, h_i].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        wantf = (want[t_i, h_i].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(wantf), 2.0 ** -126))) - 7)
        slack = ulp + 2 * W_RTOL * mag + w.k * 2.0 ** -23 * mag
        n_bad = int((np.abs(gotf - wantf) > slack).sum())
    say(f"  pipeline {name}: max ulp {int(d.max())}, >1 ulp {int(t_i.size)}, outside bound {n_bad}")
    assert n_bad == 0
    assert np.allclose(wt_gpu, o.wt, rtol=W_RTOL, atol=0)
    del bufs, y, out, x, logits
    _free()


@pytest.mark.parametrize("name", ["tiny", "mixtral_prefill", "dsr1_decode"])
def test_repeat_runs_bit_identical(dev, name):
    w = W.WORKLOADS[name]
    o = OracleRun.get(w)
    logits = torch.from_numpy(o.logits).to(dev)
    x = to_dev_bf16(o.x, dev)
    res = []
    for _ in range(3):
        idx, wt = moe.moe_route_topk(logits, w.k)
        bufs = moe.moe_dispatch(x, idx, w.E, w.C, fp8=w.fp8)
        y = torch.zeros(w.E, w.C, w.H, dtype=torch.bfloat16, device=dev) if w.fp8 else bufs.recv_x
        if w.fp8:
            y.view(torch.int16).copy_(bufs.recv_x.to(torch.int16))   # codes as bf16 bit patterns
        out = moe.moe_combine(y, bufs.token_slot, wt)
        filled = torch.from_numpy(np.nonzero(o.recv_src >= 0)[0]).to(dev)
        rows = bufs.recv_x.view(w.E * w.C, -1).index_select(0, filled)
        parts = [idx, wt, bufs.token_slot, bufs.expert_counts, rows, out]
        if w.fp8:
            parts.append(bufs.recv_scales.view(w.E * w.C, -1).index_select(0, filled))
        res.append([t.contiguous().view(torch.uint8).cpu().numpy().tobytes() for t in parts])
    assert res[0] == res[1] == res[2]
