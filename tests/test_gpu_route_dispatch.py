"""GPU parity of moe_route_dispatch (router top-k and fixed-slot dispatch in
one call; for E <= 8, and for E > 8 at moderate batch sizes, the count step
is folded into the router kernel as 32-token membership words), through the
C ABI.

Every output must equal the CPU oracle (ids, counts, slots, sources, rows
bit for bit; weights within the router tolerance) and must be bit-identical
to the separate moe_route_topk + moe_dispatch calls.  Cases: the five
workloads (E = 8 on the fused path, E = 128 and 256 on the three-step path),
E > 8 on the router-words path (every router lane layout, the 16-token
halves, the load limit on both sides),
token counts around the 32-token word and 256-token chunk boundaries, every
E <= 8 with every k, capacity overflow, fp8 rows, and token counts past the
fused path's limit; batches of at most 256 tokens with E <= 8 take a single
launch in which every pack work-group routes the batch itself.  The same
cases for moe_route_dispatch_packed against
the oracle's packed, count-sized layout and moe_route_topk +
moe_dispatch_packed.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
import oracle
import workloads as W
from gpu_common import OracleRun, W_RTOL, bf16_ulp_distance, dev_bits, require_gpu, say, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _run_both(dev, logits, x_bits, k, C, fp8):
    T, E = logits.shape
    lg = torch.from_numpy(logits).to(dev)
    xd = to_dev_bf16(x_bits, dev)
    i1, w1, b1 = moe.moe_route_dispatch(lg, xd, k, C, fp8=fp8)
    i2, w2 = moe.moe_route_topk(lg, k)
    b2 = moe.moe_dispatch(xd, i2, E, C, fp8=fp8)
    return (i1, w1, b1), (i2, w2, b2)


def _check(label, logits, x_bits, k, C, fp8, fused, separate):
    T, E = logits.shape
    H = x_bits.shape[1]
    i1, w1, b1 = fused
    i2, w2, b2 = separate
    say(f"[route+dispatch] {label}: T={T} E={E} k={k} C={C} fp8={fp8}")
    idx_o, w_o = oracle.route_topk(logits, k)
    counts_o, slot_o, src_o = oracle.assign_slots(idx_o, E, C)
    np.testing.assert_array_equal(i1.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w1.cpu().numpy(), w_o, rtol=W_RTOL, atol=0)
    np.testing.assert_array_equal(b1.expert_counts.cpu().numpy(), counts_o)
    np.testing.assert_array_equal(b1.token_slot.cpu().numpy(), slot_o)
    filled = src_o >= 0
    np.testing.assert_array_equal(b1.recv_src.cpu().numpy().reshape(-1)[filled], src_o[filled])
    if fp8:
        codes = b1.recv_x.view(E * C, H).cpu().numpy()
        c_tok, s_tok = oracle.quantize_rows_fp8(x_bits)
        np.testing.assert_array_equal(codes[filled], c_tok[src_o[filled]])
        np.testing.assert_array_equal(b1.recv_scales.view(E * C, H // 128).cpu().numpy()[filled], s_tok[src_o[filled]])
    else:
        rows = dev_bits(b1.recv_x.view(E * C, H))
        np.testing.assert_array_equal(rows[filled], x_bits[src_o[filled]])
    # identical to the separate calls, bit for bit
    assert torch.equal(i1, i2) and torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(b1.expert_counts, b2.expert_counts) and torch.equal(b1.token_slot, b2.token_slot)


@pytest.mark.parametrize("name", W.ORDER)
def test_workloads(dev, name):
    w = W.WORKLOADS[name]
    o = OracleRun.get(w)
    fused, separate = _run_both(dev, o.logits, o.x, w.k, w.C, w.fp8)
    _check(name, o.logits, o.x, w.k, w.C, w.fp8, fused, separate)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 255, 256, 257, 1000, 4096, 4097, 65536, 65537])
def test_token_counts(dev, T):
    rng = np.random.default_rng(T)
    E, k, H = 8, 2, 64
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    fused, separate = _run_both(dev, logits, x, k, T, False)
    _check(f"T={T}", logits, x, k, T, False, fused, separate)


@pytest.mark.parametrize("T", [777, 200])       # router words + pack; one launch routing in every work-group
@pytest.mark.parametrize("E", [1, 2, 3, 5, 8])
def test_every_k(dev, E, T):
    rng = np.random.default_rng(100 + E + T)
    H = 128
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    for k in range(1, E + 1):
        logits = rng.integers(-2, 3, (T, E)).astype(np.float32)     # ties everywhere
        fused, separate = _run_both(dev, logits, x, k, T, k % 2 == 1 and H % 128 == 0)
        _check(f"E={E} k={k}", logits, x, k, T, k % 2 == 1, fused, separate)


@pytest.mark.parametrize("T,E,k,fp8,C", [
    (1025, 9, 1, False, 1025),    # 16-lane groups, 9 of 16 lanes real; 65 halves (the last word's upper half cleared)
    (1031, 16, 2, True, 1031),    # 16-lane groups; 65 halves
    (1040, 24, 5, False, 90),     # 32-lane groups; 65 halves; capacity overflow
    (1040, 64, 8, False, 1040),   # one token per wave, one logit per lane; 65 halves
    (2049, 100, 6, True, 2049),   # one token per wave, two logits per lane; 129 halves
    (3000, 256, 8, False, 3000),  # one token per wave, four logits per lane
    (1100, 300, 10, False, 1100), # eight logits per lane, E not a multiple of them (scalar loads); 69 halves
    (6145, 64, 2, False, 150),    # four tokens per wave (16-lane groups, four logits per lane); 385 halves; overflow
    (8192, 256, 8, True, 8192),   # the last size whose prefix stays within 32 loads per lane
    (8193, 256, 8, False, 8193),  # one token more: route, count and pack
])
def test_router_words_for_more_than_8_experts(dev, T, E, k, fp8, C):
    """E > 8 past the in-pack count (more than 1024 tokens, more than 8192
    ids, or more than 8192 mask words): the router writes each expert's 32-token
    membership words a 16-token half per work-group, in the plain router's
    lane layout for that E and T, and pack takes counts, prefixes and ranks
    from them.  Outputs must equal the oracle and the separate calls bit for
    bit (the weights too, since both calls route with the same layout)."""
    rng = np.random.default_rng(9000 + T + E + k)
    H = 256
    logits = rng.integers(-3, 4, (T, E)).astype(np.float32) + rng.standard_normal((T, E)).astype(np.float32) * 0.25
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    fused, separate = _run_both(dev, logits, x, k, C, fp8)
    _check(f"E={E} k={k}", logits, x, k, C, fp8, fused, separate)


@pytest.mark.parametrize("T", [200, 480, 3000])
def test_every_k_counted_in_pack_and_by_chunks(dev, T):
    """E > 8, every k from 1 to 16: the lanes owning one pair (64, 32, 16, 8
    or 4 of them) sum the pair's earlier counts together.  T = 200: the batch
    is counted inside pack; T = 480: inside pack for every k (16 ids per
    thread up to k = 8, 32 beyond); T = 3000: the separate call counts with
    its own launch (256-token chunks), the fused call from the router's words.  Odd k
    overflow the capacity.  The packed layout is checked on the same
    inputs."""
    E, H = 24, 128
    rng = np.random.default_rng(7000 + T)
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    for k in range(1, 17):
        logits = rng.integers(-2, 3, (T, E)).astype(np.float32)     # ties everywhere
        C = T if k % 2 == 0 else max(1, T * k // E // 2)
        fp8 = k % 4 == 1
        fused, separate = _run_both(dev, logits, x, k, C, fp8)
        _check(f"k={k}", logits, x, k, C, fp8, fused, separate)
        fused, separate = _run_both_packed(dev, logits, x, k, fp8)
        _check_packed(f"k={k}", logits, x, k, fp8, fused, separate)


@pytest.mark.parametrize("T,E,k", [(8192, 8, 8), (8193, 8, 8), (8192, 6, 5), (8193, 6, 5), (32768, 4, 4),
                                   (32769, 4, 4)])
def test_router_word_limit_by_k(dev, T, E, k):
    """E <= 8: the router's words serve while a pair's prefix takes at most 32
    L2 loads per lane for k > 4 (8192 tokens at eight lanes per pair) and 64
    for k <= 4 (32768 tokens at 16 lanes): both sides of each limit, fixed
    slots and packed layout."""
    rng = np.random.default_rng(T + 10 * E + k)
    H = 64
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    fused, separate = _run_both(dev, logits, x, k, T, False)
    _check(f"E={E} k={k}", logits, x, k, T, False, fused, separate)
    fused, separate = _run_both_packed(dev, logits, x, k, False)
    _check_packed(f"E={E} k={k}", logits, x, k, False, fused, separate)


@pytest.mark.parametrize("T,C", [(3000, 300), (200, 20)])
def test_capacity_overflow(dev, T, C):
    rng = np.random.default_rng(9 + T)
    E, k, H = 8, 2, 256
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 3] += 2.0                                              # a hot expert overflows
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    for fp8 in (False, True):
        fused, separate = _run_both(dev, logits, x, k, C, fp8)
        _check(f"overflow fp8={fp8}", logits, x, k, C, fp8, fused, separate)


def test_empty(dev):
    lg = torch.empty(0, 8, device=dev)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    i, w, b = moe.moe_route_dispatch(lg, x, 2, 4)
    assert (b.expert_counts.cpu().numpy() == 0).all()



def test_largest_batch(dev):
    """MOE_MAX_TOKENS (2^24) tokens through route + dispatch + combine: ids,
    weights, counts, every slot and every filled source against the oracle;
    rows and combined sums on a sample.  Past 256 chunks the chunk counts are
    scanned into prefixes once, so each pair's slot costs one load whatever
    the batch."""
    T, E, k, H = 1 << 24, 8, 2, 8
    C = T // 2                     # about 2^22 tokens per expert: nothing dropped
    rng = np.random.default_rng(24)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)).to(torch.bfloat16))
    say(f"[route+dispatch] largest batch T={T} E={E} k={k} H={H} C={C}")
    idx, wt, b = moe.moe_route_dispatch(torch.from_numpy(logits).to(dev), to_dev_bf16(x, dev), k, C)
    idx_o, w_o = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    wt_h = wt.cpu().numpy()
    np.testing.assert_allclose(wt_h, w_o, rtol=W_RTOL, atol=0)
    counts_o, slot_o, src_o = oracle.assign_slots(idx_o, E, C)
    np.testing.assert_array_equal(b.expert_counts.cpu().numpy(), counts_o)
    np.testing.assert_array_equal(b.token_slot.cpu().numpy(), slot_o)
    filled = np.nonzero(src_o >= 0)[0]
    np.testing.assert_array_equal(b.recv_src.cpu().numpy().reshape(-1)[filled], src_o[filled])
    pick = filled[rng.integers(0, filled.size, 4096)]
    rows = dev_bits(b.recv_x.view(E * C, H)[torch.from_numpy(pick).to(dev)])
    np.testing.assert_array_equal(rows, x[src_o[pick]])
    out = moe.moe_combine(b.recv_x, b.token_slot, wt)    # identity experts
    tp = np.unique(np.concatenate([np.arange(64), np.arange(T - 64, T), rng.integers(0, T, 4096)]))
    want = oracle.combine(np.repeat(x[tp], k, axis=0), slot_o[tp], wt_h[tp])
    got = dev_bits(out[torch.from_numpy(tp).to(dev)])
    assert bf16_ulp_distance(got, want).max() <= 1


def test_largest_batch_packed(dev):
    """MOE_MAX_TOKENS tokens into the packed layout: offsets, every slot and
    source against the oracle; rows and combined sums on a sample."""
    T, E, k, H = 1 << 24, 8, 2, 8
    rng = np.random.default_rng(25)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)).to(torch.bfloat16))
    say(f"[route+dispatch packed] largest batch T={T} E={E} k={k} H={H}")
    idx, wt, p = moe.moe_route_dispatch_packed(torch.from_numpy(logits).to(dev), to_dev_bf16(x, dev), k)
    idx_o, _ = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    offs_o, slot_o, src_o = oracle.assign_packed(idx_o, E)
    np.testing.assert_array_equal(p.expert_offsets.cpu().numpy(), offs_o)
    np.testing.assert_array_equal(p.token_slot.cpu().numpy(), slot_o)
    np.testing.assert_array_equal(p.recv_src.cpu().numpy().reshape(-1)[:T * k], src_o)
    pick = rng.integers(0, T * k, 4096)
    rows = dev_bits(p.recv_x[torch.from_numpy(pick).to(dev)])
    np.testing.assert_array_equal(rows, x[src_o[pick]])
    out = moe.moe_combine(p.recv_x, p.token_slot, wt)
    tp = np.unique(np.concatenate([np.arange(64), np.arange(T - 64, T), rng.integers(0, T, 4096)]))
    want = oracle.combine(np.repeat(x[tp], k, axis=0), slot_o[tp], wt.cpu().numpy()[tp])
    assert bf16_ulp_distance(dev_bits(out[torch.from_numpy(tp).to(dev)]), want).max() <= 1


# ---- moe_route_dispatch_packed ----

def _run_both_packed(dev, logits, x_bits, k, fp8):
    T, E = logits.shape
    lg = torch.from_numpy(logits).to(dev)
    xd = to_dev_bf16(x_bits, dev)
    i1, w1, b1 = moe.moe_route_dispatch_packed(lg, xd, k, fp8=fp8)
    i2, w2 = moe.moe_route_topk(lg, k)
    b2 = moe.moe_dispatch_packed(xd, i2, E, fp8=fp8)
    return (i1, w1, b1), (i2, w2, b2)


def _check_packed(label, logits, x_bits, k, fp8, fused, separate):
    T, E = logits.shape
    H = x_bits.shape[1]
    i1, w1, b1 = fused
    i2, w2, b2 = separate
    say(f"[route+dispatch packed] {label}: T={T} E={E} k={k} fp8={fp8}")
    idx_o, w_o = oracle.route_topk(logits, k)
    offs_o, slot_o, src_o = oracle.assign_packed(idx_o, E)
    np.testing.assert_array_equal(i1.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w1.cpu().numpy(), w_o, rtol=W_RTOL, atol=0)
    np.testing.assert_array_equal(b1.expert_offsets.cpu().numpy(), offs_o)
    np.testing.assert_array_equal(b1.token_slot.cpu().numpy(), slot_o)
    np.testing.assert_array_equal(b1.recv_src.cpu().numpy().reshape(-1)[:T * k], src_o)
    if fp8:
        c_tok, s_tok = oracle.quantize_rows_fp8(x_bits)
        np.testing.assert_array_equal(b1.recv_x.cpu().numpy(), c_tok[src_o])
        np.testing.assert_array_equal(b1.recv_scales.cpu().numpy(), s_tok[src_o])
    else:
        np.testing.assert_array_equal(dev_bits(b1.recv_x), x_bits[src_o])
    # identical to the separate calls, bit for bit
    assert torch.equal(i1, i2) and torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(b1.expert_offsets, b2.expert_offsets) and torch.equal(b1.token_slot, b2.token_slot)
    assert torch.equal(b1.recv_src, b2.recv_src) and torch.equal(b1.recv_x.view(torch.uint8), b2.recv_x.view(torch.uint8))
    if fp8:
        assert torch.equal(b1.recv_scales.view(torch.int32), b2.recv_scales.view(torch.int32))


@pytest.mark.parametrize("name", W.ORDER)
def test_packed_workloads(dev, name):
    w = W.WORKLOADS[name]
    o = OracleRun.get(w)
    fused, separate = _run_both_packed(dev, o.logits, o.x, w.k, w.fp8)
    _check_packed(name, o.logits, o.x, w.k, w.fp8, fused, separate)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 255, 256, 257, 1000, 65536, 65537])
def test_packed_token_counts(dev, T):
    rng = np.random.default_rng(T + 7)
    E, k, H = 8, 2, 64
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    fused, separate = _run_both_packed(dev, logits, x, k, False)
    _check_packed(f"T={T}", logits, x, k, False, fused, separate)


@pytest.mark.parametrize("T,E", [(8192, 8), (8193, 8), (20000, 3), (21856, 3), (4000, 5)])
def test_packed_router_word_limit(dev, T, E):
    """E <= 8 past one chunk: each pack work-group totals the router's
    32-token membership words itself while there are at most 2048 of them
    (E * ceil(T/32)), else one work-group does it first.  Both sides of the
    limit, and words of several experts in one thread when E < 8."""
    rng = np.random.default_rng(T * 10 + E)
    k, H = 2, 64
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    fused, separate = _run_both_packed(dev, logits, x, k, False)
    _check_packed(f"T={T} E={E}", logits, x, k, False, fused, separate)


@pytest.mark.parametrize("T", [777, 200])
@pytest.mark.parametrize("E", [1, 3, 8])
def test_packed_every_k(dev, E, T):
    rng = np.random.default_rng(200 + E + T)
    H = 128
    x = W.bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))
    for k in range(1, E + 1):
        logits = rng.integers(-2, 3, (T, E)).astype(np.float32)     # ties everywhere
        fused, separate = _run_both_packed(dev, logits, x, k, k % 2 == 1)
        _check_packed(f"E={E} k={k}", logits, x, k, k % 2 == 1, fused, separate)


def test_packed_empty(dev):
    lg = torch.empty(0, 8, device=dev)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    i, w, b = moe.moe_route_dispatch_packed(lg, x, 2)
    assert (b.expert_offsets.cpu().numpy() == 0).all()
