"""moe_route_dispatch_noalloc (the library's static scratch in place of a
caller-allocated workspace) against moe_route_dispatch, through the C ABI.

Every output must be bit-identical to moe_route_dispatch's on the same
inputs.  The calls run back to back on one stream with shrinking batches, so
each later call finds the previous call's data still in the scratch array.
The shapes take every path that uses the workspace: router membership words
(E <= 8), chunk histograms with in-chunk ranks (E > 8), and the chunk scan
past 256 chunks; one batch needs more than the scratch and must be refused
before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
from gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu

# (T, H, E, k, fp8): large first, then smaller, so later calls reuse stale scratch
CASES = [
    (70_000, 128, 16, 2, False),    # 274 chunks: count, chunk scan, pack
    (4096, 1024, 64, 6, True),      # count + pack, fp8 rows
    (3000, 512, 8, 2, False),       # router membership words
    (1000, 256, 64, 8, True),       # count + pack
    (300, 256, 8, 1, False),        # router words, a few chunks
]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _inputs(T, H, E, seed, dev):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    logits = torch.randn(T, E, generator=g, dtype=torch.float32)
    logits[:, : max(1, E // 8)] += 1.0           # a few hot experts
    x = torch.randn(T, H, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return logits.to(dev), x.to(dev)


def _filled_rows(bufs, counts, C, H):
    rows = []
    for e, n in enumerate(counts.tolist()):
        rows.extend(range(e * C, e * C + min(n, C)))
    return torch.tensor(rows, dtype=torch.int64, device=bufs.recv_x.device)


def _same(a, b, what):
    assert torch.equal(a, b), what


def _run_pair(dev, T, H, E, k, fp8, seed):
    say(f"[noalloc] T={T} H={H} E={E} k={k} fp8={fp8}")
    C = T
    logits, x = _inputs(T, H, E, seed, dev)
    ref_idx, ref_w, ref = moe.moe_route_dispatch(logits, x, k, C, fp8=fp8)
    bufs = moe.DispatchBuffers.allocate(T, H, E, k, C, fp8, dev, workspace=False)
    # outputs poisoned so that anything left unwritten shows
    bufs.token_slot.fill_(-7)
    bufs.expert_counts.fill_(-7)
    idx, w, bufs = moe.moe_route_dispatch_noalloc(logits, x, k, C, fp8=fp8, bufs=bufs)
    torch.cuda.synchronize()
    _same(idx, ref_idx, "topk_idx")
    _same(w.view(torch.int32), ref_w.view(torch.int32), "topk_w")
    _same(bufs.expert_counts, ref.expert_counts, "expert_counts")
    _same(bufs.token_slot, ref.token_slot, "token_slot")
    assert int(bufs.expert_counts.sum()) == T * k
    rows = _filled_rows(bufs, ref.expert_counts.cpu(), C, H)
    _same(bufs.recv_src.view(-1).index_select(0, rows), ref.recv_src.view(-1).index_select(0, rows), "recv_src")
    rx = bufs.recv_x.view(E * C, -1).index_select(0, rows)
    rr = ref.recv_x.view(E * C, -1).index_select(0, rows)
    _same(rx.view(torch.uint8), rr.view(torch.uint8), "recv_x")
    if fp8:
        a = bufs.recv_scales.view(E * C, -1).index_select(0, rows)
        b = ref.recv_scales.view(E * C, -1).index_select(0, rows)
        _same(a.view(torch.int32), b.view(torch.int32), "recv_scales")
    say(f"  identical ({rows.numel()} filled rows)")


def test_noalloc_matches_route_dispatch_in_sequence(dev):
    for i, (T, H, E, k, fp8) in enumerate(CASES):
        _run_pair(dev, T, H, E, k, fp8, seed=500 + i)


def test_noalloc_two_calls_second_smaller(dev):
    """Two calls in a row on the same stream with no synchronisation between
    them, the second smaller, each checked against moe_route_dispatch."""
    (T1, H1, E1, k1, f1), (T2, H2, E2, k2, f2) = (6000, 256, 32, 4, False), (700, 256, 32, 4, False)
    l1, x1 = _inputs(T1, H1, E1, 11, dev)
    l2, x2 = _inputs(T2, H2, E2, 12, dev)
    b1 = moe.DispatchBuffers.allocate(T1, H1, E1, k1, T1, f1, dev, workspace=False)
    b2 = moe.DispatchBuffers.allocate(T2, H2, E2, k2, T2, f2, dev, workspace=False)
    i1, w1, _ = moe.moe_route_dispatch_noalloc(l1, x1, k1, T1, bufs=b1)
    i2, w2, _ = moe.moe_route_dispatch_noalloc(l2, x2, k2, T2, bufs=b2)
    r1 = moe.moe_route_dispatch(l1, x1, k1, T1)
    r2 = moe.moe_route_dispatch(l2, x2, k2, T2)
    torch.cuda.synchronize()
    for got, ref, idx, ref_idx in ((b1, r1[2], i1, r1[0]), (b2, r2[2], i2, r2[0])):
        _same(idx, ref_idx, "topk_idx")
        _same(got.expert_counts, ref.expert_counts, "expert_counts")
        _same(got.token_slot, ref.token_slot, "token_slot")


def test_noalloc_refuses_batches_beyond_its_scratch(dev):
    T, H, E, k = 140_000, 128, 16, 8
    assert moe.moe_dispatch_workspace_bytes(T, E, k) > moe.MOE_NOALLOC_SCRATCH_BYTES
    logits, x = _inputs(T, H, E, 3, dev)
    bufs = moe.DispatchBuffers.allocate(T, H, E, k, 8, False, dev, workspace=False)
    bufs.token_slot.fill_(-7)
    with pytest.raises(moe.MoeError) as err:
        moe.moe_route_dispatch_noalloc(logits, x, k, 8, bufs=bufs)
    assert err.value.status == moe.binding.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert int((bufs.token_slot != -7).sum()) == 0, "a refused call must enqueue nothing"


@pytest.mark.parametrize("T,H,E,k,fp8", [(2048, 512, 8, 2, False), (1000, 256, 64, 8, True)])
def test_noalloc_graph_replays(dev, T, H, E, k, fp8):
    """The case the entry point exists for: route + dispatch captured in a
    HIP graph with no workspace to allocate, replayed several times.  Between
    replays an eager call on a different batch overwrites the library's
    scratch; every replay must still reproduce the eager outputs bit for bit
    (nothing in the scratch is carried from one call to the next)."""
    say(f"[noalloc graph] T={T} H={H} E={E} k={k} fp8={fp8}")
    logits, x = _inputs(T, H, E, 21, dev)
    other_l, other_x = _inputs(3000, 128, 16, 22, dev)
    C = T
    bufs = moe.DispatchBuffers.allocate(T, H, E, k, C, fp8, dev, workspace=False)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    wt = torch.empty(T, k, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    outs = (idx, wt, bufs.expert_counts, bufs.token_slot, bufs.recv_src)

    def clear():
        for t in outs:
            t.zero_()

    clear()
    torch.cuda.synchronize()
    moe.moe_route_dispatch_noalloc(logits, x, k, C, fp8=fp8, bufs=bufs, topk_idx=idx, topk_w=wt, stream=side)
    side.synchronize()
    ref = [t.clone() for t in outs]
    rows = _filled_rows(bufs, bufs.expert_counts.cpu(), C, H)
    ref_rows = bufs.recv_x.view(E * C, -1).index_select(0, rows).clone()
    r_idx, r_w, r_bufs = moe.moe_route_dispatch(logits, x, k, C, fp8=fp8)
    torch.cuda.synchronize()
    _same(ref[0], r_idx, "topk_idx")
    _same(ref[3], r_bufs.token_slot, "token_slot")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        moe.moe_route_dispatch_noalloc(logits, x, k, C, fp8=fp8, bufs=bufs, topk_idx=idx, topk_w=wt, stream=side)
    for rep in range(4):
        clear()
        bufs.recv_x.view(torch.uint8)[0].fill_(0)
        moe.moe_route_dispatch_noalloc(other_l, other_x, 4, 3000)      # eager, different batch: scratch reused
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"
        got_rows = bufs.recv_x.view(E * C, -1).index_select(0, rows)
        assert torch.equal(got_rows.view(torch.uint8), ref_rows.view(torch.uint8)), f"replay {rep} rows differ"
