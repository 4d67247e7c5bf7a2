"""GPU parity on edge cases and random small shapes: empty and one-token
batches, ragged token counts (not a multiple of the 256-token count chunk)
and ragged hidden sizes (not a multiple of the 64-lane x 16-byte row
stride), planted ties and signed zeros, k = E, the largest E and k,
capacity overflow, out-of-range expert ids, fp8 special blocks, and canary
checks that nothing outside the defined outputs is written.
Every expected value comes from the CPU oracle."""
import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
import oracle
import workloads as W
from gpu_common import W_RTOL, bf16_ulp_distance, dev_bits, require_gpu, say, to_dev_bf16

pytestmark = pytest.mark.gpu

SENT = -123456789          # int32 canary
SENT_BF16 = 0x7FBD         # a NaN pattern no kernel writes


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    return W.bits(torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16))


def _logits(rng, T, E, kind):
    if kind == "normal":
        return rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        return rng.integers(-3, 4, (T, E)).astype(np.float32)
    if kind == "zeros":
        return rng.choice(np.array([0.0, -0.0, 0.5, -0.5], np.float32), (T, E))
    if kind == "equal":
        return np.full((T, E), 0.25, np.float32)
    raise ValueError(kind)


def run_case(dev, T, H, E, k, C, fp8, kind="normal", seed=0, idx_override=None):
    """Route, dispatch and combine a random case on the GPU and compare every
    output with the oracle.  Returns the GPU dispatch buffers."""
    say(f"[case] T={T} H={H} E={E} k={k} C={C} fp8={fp8} logits={kind} seed={seed}")
    rng = np.random.default_rng(seed)
    logits = _logits(rng, T, E, kind)
    x = _bf16_bits(rng.standard_normal((T, H)) * rng.choice([1e-3, 1.0, 30.0], (T, 1)))
    # route
    if T > 0:
        idx_g, w_g = moe.moe_route_topk(torch.from_numpy(logits).to(dev), k)
        idx_o, w_o = oracle.route_topk(logits, k)
        np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)
        np.testing.assert_allclose(w_g.cpu().numpy(), w_o, rtol=W_RTOL, atol=0)
    else:
        idx_o = np.zeros((0, k), np.int32)
        w_o = np.zeros((0, k), np.float32)
    if idx_override is not None:
        idx_o = idx_override
    # dispatch (oracle ids in, so dispatch is checked on its own)
    bufs = moe.DispatchBuffers.allocate(T, H, E, k, C, fp8, dev)
    bufs.recv_src.fill_(SENT)
    bufs.token_slot.fill_(SENT)
    bufs.expert_counts.fill_(SENT)
    if fp8:
        bufs.recv_x.fill_(0xA5)
        bufs.recv_scales.fill_(-7.0)
    else:
        bufs.recv_x.view(torch.int16).fill_(SENT_BF16)
    moe.moe_dispatch(to_dev_bf16(x, dev), torch.from_numpy(np.ascontiguousarray(idx_o)).to(dev), E, C, fp8=fp8,
                     bufs=bufs)
    if idx_override is None:
        counts_o, slot_o, src_o = oracle.assign_slots(idx_o, E, C)
    else:
        counts_o, slot_o, src_o = _assign_with_invalid(idx_o, E, C)
    np.testing.assert_array_equal(bufs.expert_counts.cpu().numpy(), counts_o)
    np.testing.assert_array_equal(bufs.token_slot.cpu().numpy(), slot_o)
    src_g = bufs.recv_src.cpu().numpy().reshape(-1)
    filled = src_o >= 0
    np.testing.assert_array_equal(src_g[filled], src_o[filled])
    assert (src_g[~filled] == SENT).all(), "an unfilled recv_src slot was written"
    if fp8:
        codes = bufs.recv_x.view(E * C, H).cpu().numpy()
        scales = bufs.recv_scales.view(E * C, H // 128).cpu().numpy()
        if T > 0:
            c_tok, s_tok = oracle.quantize_rows_fp8(x)
            np.testing.assert_array_equal(codes[filled], c_tok[src_o[filled]])
            np.testing.assert_array_equal(scales[filled], s_tok[src_o[filled]])
        assert (codes[~filled] == 0xA5).all() and (scales[~filled] == -7.0).all()
    else:
        rows = dev_bits(bufs.recv_x.view(E * C, H))
        np.testing.assert_array_equal(rows[filled], x[src_o[filled]])
        assert (rows[~filled] == SENT_BF16).all(), "an unfilled recv_x slot was written"
    # combine on seeded expert outputs placed at the oracle's slots
    if T > 0:
        y_pairs = _bf16_bits(rng.standard_normal((T * k, H)))
        y = torch.empty(E, C, H, dtype=torch.bfloat16, device=dev)
        y.view(torch.int16).fill_(SENT_BF16)
        flat = slot_o.reshape(-1)
        keep = np.nonzero(flat >= 0)[0]
        if keep.size:
            y.view(-1, H).index_copy_(0, torch.from_numpy(flat[keep].astype(np.int64)).to(dev),
                                      to_dev_bf16(y_pairs[keep], dev))
        out = torch.empty(T + 1, H, dtype=torch.bfloat16, device=dev)
        out.view(torch.int16).fill_(SENT_BF16)
        moe.moe_combine(y, torch.from_numpy(slot_o).to(dev), torch.from_numpy(w_o).to(dev), out=out[:T])
        got = dev_bits(out)
        want = oracle.combine(y_pairs, slot_o, w_o)
        d = bf16_ulp_distance(got[:T], want)
        assert d.max(initial=0) <= 1
        assert (got[T] == SENT_BF16).all(), "combine wrote past its output"
    return bufs


def _assign_with_invalid(idx, E, C):
    """Oracle slots when some ids are out of range: those pairs are dropped
    and not counted.  They are renamed to a spare expert E, given to the
    oracle with E + 1 experts (slot e*C + r is the same for e < E), and then
    discarded."""
    valid = (idx >= 0) & (idx < E)
    ext = np.where(valid, idx, E).astype(np.int32)
    counts_x, slot_x, src_x = oracle.assign_slots(ext, E + 1, C)
    slot = np.where(valid, slot_x, -1).astype(np.int32)
    return counts_x[:E].copy(), slot, src_x[: E * C].copy()


@pytest.mark.parametrize("fp8", [False, True])
def test_empty_batch(dev, fp8):
    bufs = run_case(dev, 0, 128, 8, 2, 4, fp8)
    assert (bufs.expert_counts.cpu().numpy() == 0).all()


def test_empty_combine_and_route(dev):
    out = moe.moe_combine(torch.empty(2, 2, 64, dtype=torch.bfloat16, device=dev),
                          torch.empty(0, 2, dtype=torch.int32, device=dev),
                          torch.empty(0, 2, dtype=torch.float32, device=dev))
    assert out.shape == (0, 64)
    idx, w = moe.moe_route_topk(torch.empty(0, 8, dtype=torch.float32, device=dev), 2)
    assert idx.shape == (0, 2)


@pytest.mark.parametrize("T,H,E,k,C,fp8,kind", [
    (1, 8, 1, 1, 1, False, "normal"),
    (1, 128, 1, 1, 1, True, "normal"),
    (257, 136, 16, 4, 257, False, "normal"),      # ragged T and H
    (1000, 8 * 65, 24, 3, 1000, False, "ties"),
    (513, 384, 40, 6, 513, True, "zeros"),
    (300, 256, 16, 16, 300, False, "normal"),     # k = E
    (64, 128, 1024, 16, 64, True, "normal"),      # largest E and k
    (70, 1024, 1024, 16, 70, False, "ties"),
    (200, 640, 8, 2, 200, False, "equal"),        # all-equal logits
    (129, 7168, 256, 8, 129, True, "normal"),
    (4100, 64, 64, 8, 4100, False, "normal"),     # many chunks
    # grids large enough to keep each pack split (bf16 aims at 8/k vectors per lane)
    (4096, 4096, 8, 1, 4096, False, "normal"),    # 8 vectors per lane
    (4096, 2056, 16, 2, 4096, False, "normal"),   # 4, ragged last segment
    (3000, 2056, 16, 3, 3000, False, "ties"),     # 2, ragged
    (2500, 1024, 64, 4, 2500, False, "normal"),   # 2
    (2300, 1024, 32, 1, 2300, True, "normal"),    # fp8: 2 groups per lane
    # 257-1024 tokens counted inside pack (ids <= 8192, 32 per thread past 4096; masks <= 8192 words), and past
    # each limit
    (300, 7168, 256, 8, 300, True, "normal"),
    (512, 2048, 64, 8, 512, False, "ties"),
    (1024, 256, 64, 4, 1024, False, "ties"),      # 4096 ids, 64 experts x 32 words: the largest local batch
    (800, 512, 128, 2, 800, True, "normal"),      # 128 experts x 25 words
    (1025, 256, 64, 4, 1025, False, "normal"),    # one token past the limit: count launch
    (1000, 128, 130, 4, 1000, False, "zeros"),    # 130 experts x 32 words
    (1000, 128, 257, 4, 1000, False, "ties"),     # 257 experts x 32 words: count launch
    (1024, 64, 32, 5, 300, False, "normal"),      # 5120 ids: count launch, capacity overflow
    (500, 256, 256, 8, 500, False, "normal"),     # 256 experts x 16 words
    (500, 256, 512, 8, 500, False, "normal"),     # 512 experts x 16 words: the largest local mask
    (500, 256, 520, 8, 500, False, "normal"),     # 520 experts x 16 words: count launch
    (400, 128, 1024, 8, 400, False, "zeros"),     # 1024 experts: count launch
    (1100, 64, 1024, 16, 1100, False, "normal"),  # the largest E and k together through the count launch
    (2000, 64, 1024, 16, 700, False, "ties"),     # and with ties and capacity overflow
    (512, 64, 32, 16, 512, False, "normal"),      # 8192 ids: the most, 32 per thread
    (257, 64, 16, 16, 257, False, "normal"),      # 4112 ids: 32 per thread
    (520, 64, 32, 16, 520, False, "ties"),        # 8320 ids: count launch
    (1024, 256, 256, 8, 1024, False, "ties"),     # 8192 ids and 8192 mask words together
    (600, 7168, 256, 8, 600, True, "normal"),     # a mid-size batch of the DeepSeek-R1 shape, 4800 ids
    (480, 136, 20, 3, 37, False, "normal"),       # counted inside pack, with capacity overflow
    # more than 256 chunks: the chunk counts are scanned into prefixes first
    (66000, 64, 16, 4, 66000, False, "normal"),
    (65800, 128, 24, 2, 65800, True, "ties"),
    (70000, 8, 4, 2, 20000, False, "normal"),     # and capacity overflow on that path
])
def test_shapes(dev, T, H, E, k, C, fp8, kind):
    run_case(dev, T, H, E, k, C, fp8, kind)


@pytest.mark.parametrize("fp8", [False, True])
def test_capacity_overflow(dev, fp8):
    # all-equal logits send every token to experts 0..k-1: capacity 37 < T
    bufs = run_case(dev, 300, 256, 8, 2, 37, fp8, kind="equal")
    counts = bufs.expert_counts.cpu().numpy()
    assert counts[0] == 300 and counts[1] == 300 and (counts[2:] == 0).all()
    ts = bufs.token_slot.cpu().numpy()
    assert (ts[37:] == -1).all() and (ts[:37, 0] == np.arange(37)).all()


def test_out_of_range_ids_are_dropped(dev):
    rng = np.random.default_rng(9)
    T, E, k = 90, 12, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[5, 1] = -1
    idx[17, 0] = E
    idx[40, 2] = 1 << 30
    idx[41, 2] = -(1 << 30)
    run_case(dev, T, 64, E, k, T, False, idx_override=idx)


def test_random_small_shapes(dev):
    rng = np.random.default_rng(2025)
    for case in range(24):
        E = int(rng.integers(1, 300))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.integers(1, 300))
        fp8 = bool(rng.integers(0, 2))
        H = 128 * int(rng.integers(1, 6)) if fp8 else 8 * int(rng.integers(1, 80))
        C = int(rng.integers(max(1, T // 4), T + 1))
        kind = ["normal", "ties", "zeros"][case % 3]
        run_case(dev, T, H, E, k, C, fp8, kind, seed=case)


def test_fp8_special_blocks(dev):
    T, H, E, k = 8, 512, 4, 2
    vals = np.zeros((T, H), np.float32)
    vals[1, :] = -0.0                                   # negative zeros
    vals[2, 0] = 3e38                                   # one huge element
    vals[2, 1:128] = 1.0
    vals[3, :] = 1e-38                                  # tiny (fp32 subnormal range after scaling)
    vals[4, ::2] = 448.0
    vals[4, 1::2] = -1e-4
    vals[5] = np.random.default_rng(1).standard_normal(H) * 1e4
    vals[6, :128] = 2.0 ** -133                          # bf16 subnormal
    vals[7] = np.linspace(-1, 1, H)
    x = _bf16_bits(vals)
    idx = np.array([[t % E, (t + 1) % E] for t in range(T)], np.int32)
    bufs = moe.moe_dispatch(to_dev_bf16(x, dev), torch.from_numpy(idx).to(dev), E, T, fp8=True)
    counts, slot, src = oracle.assign_slots(idx, E, T)
    np.testing.assert_array_equal(bufs.token_slot.cpu().numpy(), slot)
    c_tok, s_tok = oracle.quantize_rows_fp8(x)
    codes = bufs.recv_x.view(E * T, H).cpu().numpy()
    scales = bufs.recv_scales.view(E * T, H // 128).cpu().numpy()
    filled = src >= 0
    np.testing.assert_array_equal(codes[filled], c_tok[src[filled]])
    np.testing.assert_array_equal(scales[filled], s_tok[src[filled]])


def test_api_rejects_bad_arguments(dev):
    lib = moe.load()
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device=dev)
    logits = torch.zeros(4, 8, dtype=torch.float32, device=dev)
    idx = torch.zeros(4, 2, dtype=torch.int32, device=dev)
    w = torch.zeros(4, 2, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    assert lib.moe_route_topk(logits.data_ptr(), 4, 8, 9, idx.data_ptr(), w.data_ptr(), s) == moe.binding.MOE_ERR_INVALID
    assert lib.moe_route_topk(logits.data_ptr(), 4, 2000, 2, idx.data_ptr(), w.data_ptr(), s) == \
        moe.binding.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk(None, 4, 8, 2, idx.data_ptr(), w.data_ptr(), s) == moe.binding.MOE_ERR_INVALID
    bufs = moe.DispatchBuffers.allocate(4, 64, 8, 2, 4, False, dev)
    args = [x.data_ptr(), 4, 64, idx.data_ptr(), 8, 2, 4, 0, bufs.recv_x.data_ptr(), None, bufs.recv_src.data_ptr(),
            bufs.expert_counts.data_ptr(), bufs.token_slot.data_ptr(), bufs.workspace.data_ptr(),
            bufs.workspace.numel(), s]
    assert lib.moe_dispatch(*args) == 0
    bad = list(args); bad[13] = None
    assert lib.moe_dispatch(*bad) == moe.binding.MOE_ERR_WORKSPACE
    bad = list(args); bad[14] = 16
    assert lib.moe_dispatch(*bad) == moe.binding.MOE_ERR_WORKSPACE
    bad = list(args); bad[2] = 60
    assert lib.moe_dispatch(*bad) == moe.binding.MOE_ERR_UNSUPPORTED
    bad = list(args); bad[7] = 1                     # fp8 needs H % 128 == 0
    assert lib.moe_dispatch(*bad) == moe.binding.MOE_ERR_UNSUPPORTED
    bad = list(args); bad[0] = x.data_ptr() + 2      # misaligned
    assert lib.moe_dispatch(*bad) == moe.binding.MOE_ERR_INVALID
    bad = list(args); bad[6] = 0
    assert lib.moe_dispatch(*bad) == moe.binding.MOE_ERR_INVALID
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,H,k", [
    (4096, 2056, 3),    # one work-group per token, 320 threads for a ragged 257-vector row
    (2048, 8192, 2),    # one work-group per token, 1024 threads
    (4100, 8, 5),       # one-vector rows: 64-thread groups with 63 idle lanes
    (16384, 4096, 1),   # 512-vector segments tile the row and there are many waves: segmented launch
    (2500, 16392, 2),   # rows past 1024 vectors: segmented launch, last segment one vector long
    (100, 7168, 8),     # few tokens: one vector per lane, segmented launch
])
def test_combine_launch_shapes_with_dropped_pairs(dev, T, H, k):
    """Each of combine's launch shapes with dropped pairs mixed in: slot -1,
    slots at or past E*C (both skipped), and a token whose pairs are all
    dropped (its output is +0)."""
    say(f"combine launch shape T={T} H={H} k={k}")
    rng = np.random.default_rng(T + H + k)
    R = T * k
    slot = rng.permutation(R).astype(np.int32).reshape(T, k)
    drop = rng.random((T, k)) < 0.03
    past = rng.random((T, k)) < 0.01
    slot[drop] = -1
    slot[past] = (R + rng.integers(0, 1 << 30, int(past.sum()))).astype(np.int32)
    slot[T // 2, :] = -1
    w = rng.uniform(-1, 1, (T, k)).astype(np.float32)
    y = torch.randn(1, R, H, device=dev).to(torch.bfloat16)
    out = torch.empty(T + 1, H, dtype=torch.bfloat16, device=dev)
    out.view(torch.int16).fill_(SENT_BF16)
    moe.moe_combine(y, torch.from_numpy(slot).to(dev), torch.from_numpy(w).to(dev), out=out[:T])
    got = dev_bits(out)
    kept = np.where((slot >= 0) & (slot < R), slot, -1).astype(np.int32)
    rows = dev_bits(y.view(R, H))[np.clip(kept, 0, R - 1).reshape(-1)]
    want = oracle.combine(rows, kept, w)
    assert bf16_ulp_distance(got[:T], want).max() <= 1
    assert (got[T // 2] == 0).all()
    assert (got[T] == SENT_BF16).all(), "combine wrote past its output"


def test_combine_rejects_overlapping_output(dev):
    y = torch.zeros(2, 4, 64, dtype=torch.bfloat16, device=dev)
    ts = torch.zeros(4, 1, dtype=torch.int32, device=dev)
    w = torch.ones(4, 1, dtype=torch.float32, device=dev)
    with pytest.raises(moe.MoeError):
        moe.moe_combine(y, ts, w, out=y.view(8, 64)[:4])


def test_workspace_reused_across_shapes(dev):
    """One workspace, sized for the largest call, serves a run of dispatches
    whose T, E and k differ, so each call's regions (per-chunk counts,
    in-chunk ranks) fall on words an earlier call left in another region.
    Every call must still match the oracle exactly."""
    cases = [(9000, 64, 4), (300, 256, 8), (70000, 8, 2), (256, 128, 8), (1, 1, 1), (20000, 256, 8),
             (4097, 16, 2), (9000, 64, 4)]
    ws_bytes = max(moe.moe_dispatch_workspace_bytes(T, E, k) for T, E, k in cases)
    shared = torch.full((ws_bytes,), 0x5A, dtype=torch.uint8, device=dev)
    H = 64
    for n, (T, E, k) in enumerate(cases):
        say(f"[workspace reuse] call {n}: T={T} E={E} k={k}")
        rng = np.random.default_rng(700 + n)
        idx_o, _ = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
        C = max(1, T * k // E)
        x = _bf16_bits(rng.standard_normal((T, H)))
        bufs = moe.DispatchBuffers.allocate(T, H, E, k, C, False, dev)
        bufs.workspace = shared
        moe.moe_dispatch(to_dev_bf16(x, dev), torch.from_numpy(idx_o).to(dev), E, C, bufs=bufs)
        counts_o, slot_o, src_o = oracle.assign_slots(idx_o, E, C)
        np.testing.assert_array_equal(bufs.expert_counts.cpu().numpy(), counts_o)
        np.testing.assert_array_equal(bufs.token_slot.cpu().numpy(), slot_o)
        filled = src_o >= 0
        np.testing.assert_array_equal(bufs.recv_src.cpu().numpy().reshape(-1)[filled], src_o[filled])
        rows = dev_bits(bufs.recv_x.view(E * C, H))
        np.testing.assert_array_equal(rows[filled], x[src_o[filled]])


@pytest.mark.parametrize("E", [33, 50, 64, 65, 100, 127, 128, 129, 200, 255, 256, 257, 300, 512, 513, 1000])
@pytest.mark.parametrize("kind", ["normal", "ties", "zeros"])
def test_route_lane_layouts(dev, E, kind):
    """Every lane layout of the router (16-lane groups with 4, 8 or 16
    logits per lane, or one wave with 8 or 16 per lane), aligned and ragged
    E, with ties and signed zeros: ids exact, weights within tolerance."""
    rng = np.random.default_rng(E * 3 + len(kind))
    T, k = (333 if E % 2 else 6200), min(8, E)      # both sides of the 6144-token layout switch
    logits = _logits(rng, T, E, kind)
    idx_g, w_g = moe.moe_route_topk(torch.from_numpy(logits).to(dev), k)
    idx_o, w_o = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w_g.cpu().numpy(), w_o, rtol=W_RTOL, atol=0)
