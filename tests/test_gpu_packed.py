"""GPU parity of the packed, count-sized dispatch layout
(moe_dispatch_packed; handbook "NVSHMEM and DeepEP", "High-throughput mode":
count first, then a receive buffer of exactly the needed size) and of
combine reading it, through the C ABI, against the CPU oracle.

Offsets, row indices, sources and row contents (bf16 bits, or E4M3 codes and
scales) must be identical; combine within one bf16 ulp (bit-identical
expected).  Cases: the five workloads at full size, ragged and tiny batches,
one expert, k = E, ids out of range, and canaries on the rows past the last
routed pair.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
import oracle
import workloads as W
from gpu_common import OracleRun, bf16_ulp_distance, dev_bits, require_gpu, say, to_dev_bf16

pytestmark = pytest.mark.gpu

SENT = -123456789
SENT_BF16 = 0x7FBD


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _run_packed(dev, x_bits, idx, E, fp8, label):
    T, H = x_bits.shape
    k = idx.shape[1]
    say(f"[packed] {label}: T={T} H={H} E={E} k={k} fp8={fp8}")
    bufs = moe.PackedBuffers.allocate(T, H, E, k, fp8, dev)
    bufs.recv_src.fill_(SENT)
    bufs.token_slot.fill_(SENT)
    bufs.expert_offsets.fill_(SENT)
    if fp8:
        bufs.recv_x.fill_(0xA5)
        bufs.recv_scales.fill_(-7.0)
    else:
        bufs.recv_x.view(torch.int16).fill_(SENT_BF16)
    moe.moe_dispatch_packed(to_dev_bf16(x_bits, dev), torch.from_numpy(np.ascontiguousarray(idx)).to(dev), E,
                            fp8=fp8, bufs=bufs)
    return bufs


def _expect(idx, E):
    """Oracle layout; ids outside [0, E) are renamed to a spare expert E, laid
    out after all real experts, and then dropped."""
    valid = (idx >= 0) & (idx < E)
    ext = np.where(valid, idx, E).astype(np.int32)
    offsets_x, slot_x, src_x = oracle.assign_packed(ext, E + 1)
    n = int(offsets_x[E])
    slot = np.where(valid, slot_x, -1).astype(np.int32)
    return offsets_x[:E + 1].copy(), slot, src_x[:n].copy()


def _check(bufs, x_bits, idx, E, fp8):
    T, H = x_bits.shape
    k = idx.shape[1]
    offsets, slot, src = _expect(idx, E)
    n = int(offsets[E])
    np.testing.assert_array_equal(bufs.expert_offsets.cpu().numpy(), offsets)
    np.testing.assert_array_equal(bufs.token_slot.cpu().numpy(), slot)
    src_g = bufs.recv_src.cpu().numpy()
    np.testing.assert_array_equal(src_g[:n], src)
    assert (src_g[n:T * k] == SENT).all(), "recv_src written past the last routed pair"
    if fp8:
        codes = bufs.recv_x.cpu().numpy()
        scales = bufs.recv_scales.cpu().numpy()
        if n:
            c_tok, s_tok = oracle.quantize_rows_fp8(x_bits)
            np.testing.assert_array_equal(codes[:n], c_tok[src])
            np.testing.assert_array_equal(scales[:n], s_tok[src])
        assert (codes[n:] == 0xA5).all() and (scales[n:] == -7.0).all()
    else:
        rows = dev_bits(bufs.recv_x) if T * k else np.zeros((0, H), np.uint16)
        np.testing.assert_array_equal(rows[:n], x_bits[src])
        assert (rows[n:] == SENT_BF16).all(), "recv_x written past the last routed pair"
    return slot


@pytest.mark.parametrize("name", W.ORDER)
def test_workloads_full_size(dev, name):
    w = W.WORKLOADS[name]
    o = OracleRun.get(w)
    bufs = _run_packed(dev, o.x, o.idx, w.E, w.fp8, name)
    slot = _check(bufs, o.x, o.idx, w.E, w.fp8)
    # combine reads the packed rows: expert outputs placed at the packed rows
    y_pairs = o.y_pairs
    y = torch.empty(w.T * w.k, w.H, dtype=torch.bfloat16, device=dev)
    flat = slot.reshape(-1)
    y.index_copy_(0, torch.from_numpy(flat.astype(np.int64)).to(dev), to_dev_bf16(y_pairs, dev))
    out = moe.moe_combine(y, torch.from_numpy(slot).to(dev), torch.from_numpy(o.wt).to(dev))
    got = dev_bits(out)
    want = oracle.combine(y_pairs, slot, o.wt)
    d = bf16_ulp_distance(got, want)
    say(f"  packed combine {name}: max ulp {int(d.max(initial=0))}")
    assert d.max(initial=0) <= 1
    del bufs, y, out


@pytest.mark.parametrize("T,H,E,k,fp8", [
    (1, 128, 8, 2, False), (1, 128, 8, 2, True), (255, 256, 16, 4, False), (257, 384, 16, 4, True),
    (1000, 64, 1, 1, False), (700, 128, 6, 6, True), (3000, 1024, 128, 8, False), (513, 8, 1024, 16, False),
    (5000, 2048, 256, 8, True), (70000, 64, 8, 2, False), (66000, 128, 16, 3, True),
    (400, 256, 64, 8, True), (511, 512, 300, 6, False),
])
def test_shapes(dev, T, H, E, k, fp8):
    rng = np.random.default_rng(T + H + E + k + fp8)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    bufs = _run_packed(dev, x, idx, E, fp8, "shape")
    _check(bufs, x, idx, E, fp8)


def test_out_of_range_ids_are_dropped(dev):
    rng = np.random.default_rng(12)
    T, H, E, k = 600, 128, 16, 4
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    bad = rng.random((T, k)) < 0.1
    idx[bad] = rng.choice(np.array([-1, E, E + 5, -100], np.int32), int(bad.sum()))
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    for fp8 in (False, True):
        bufs = _run_packed(dev, x, idx, E, fp8, "invalid ids")
        _check(bufs, x, idx, E, fp8)


def test_empty_batch(dev):
    for fp8 in (False, True):
        x = torch.empty(0, 128, dtype=torch.bfloat16, device=dev)
        idx = torch.empty(0, 2, dtype=torch.int32, device=dev)
        bufs = moe.PackedBuffers.allocate(0, 128, 8, 2, fp8, dev)
        bufs.expert_offsets.fill_(SENT)
        moe.moe_dispatch_packed(x, idx, 8, fp8=fp8, bufs=bufs)
        assert (bufs.expert_offsets.cpu().numpy() == 0).all()


def test_repeat_runs_bit_identical(dev):
    w = W.WORKLOADS["glm_prefill"]
    o = OracleRun.get(w)
    a = _run_packed(dev, o.x, o.idx, w.E, w.fp8, "repeat a")
    b = _run_packed(dev, o.x, o.idx, w.E, w.fp8, "repeat b")
    assert torch.equal(a.recv_x, b.recv_x) and torch.equal(a.recv_scales, b.recv_scales)
    assert torch.equal(a.token_slot, b.token_slot) and torch.equal(a.expert_offsets, b.expert_offsets)
