"""The library's calls can be captured in a HIP graph and replayed (handbook
"NVSHMEM and DeepEP", "Low-latency mode": fixed slots make every address
known on the device, so no host round trip is needed and the calls are
graph-capturable).  No call synchronises, allocates, or records a memset.

Each test captures a step on a side stream, replays the graph several times
with the program's own eager work and synchronisations in between, and
checks every replay bit for bit against the eager results of the same calls;
the eager results of the prepared calls (the ones bench.py times) are
checked against the oracle first."""
import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
import oracle
import workloads as W
from gpu_common import W_RTOL, OracleRun, bf16_ulp_distance, dev_bits, place_rows, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _outputs(bufs, idx, wt, out, extra=()):
    return [t.clone() for t in (idx, wt, bufs.token_slot, bufs.recv_src, bufs.recv_x, out, *extra)]


@pytest.mark.parametrize("name", ["tiny", "dsr1_decode", "mixtral_prefill"])
@pytest.mark.parametrize("fused", [True, False])
def test_step_graph_replays_match_eager(dev, name, fused):
    w = W.WORKLOADS[name]
    o = OracleRun.get(w)
    say(f"[graph] {name} fused_route={fused}")
    logits = torch.from_numpy(o.logits).to(dev)
    x = W.make_x(w).to(dev)
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device=dev)
    wt = torch.empty(w.T, w.k, dtype=torch.float32, device=dev)
    bufs = moe.DispatchBuffers.allocate(w.T, w.H, w.E, w.k, w.C, w.fp8, dev)
    y = place_rows(w, o.y_pairs, o.token_slot, dev)
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    step = moe.PreparedStep(logits, w.k, x, w.C, w.fp8, bufs, y, out, idx, wt, stream=side, fuse_route=fused)

    # eager reference on the same stream and buffers (outputs cleared first:
    # unfilled slots are never written, so they keep what was there)
    for t in (idx, wt, bufs.token_slot, bufs.recv_src, out):
        t.zero_()
    torch.cuda.synchronize()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.route_and_dispatch()
        step.combine()
    side.synchronize()
    ref = _outputs(bufs, idx, wt, out)
    # the prepared calls (what bench.py times) against the oracle
    np.testing.assert_array_equal(idx.cpu().numpy(), o.idx)
    np.testing.assert_allclose(wt.cpu().numpy(), o.wt, rtol=W_RTOL, atol=0)
    np.testing.assert_array_equal(bufs.token_slot.cpu().numpy(), o.token_slot)
    np.testing.assert_array_equal(bufs.expert_counts.cpu().numpy(), o.counts)
    want = oracle.combine(o.y_pairs, o.token_slot, wt.cpu().numpy())
    assert bf16_ulp_distance(dev_bits(out), want).max(initial=0) <= 1

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step.route_and_dispatch()
        step.combine()
    for rep in range(4):
        for t in (idx, wt, bufs.token_slot, bufs.recv_src, out):
            t.zero_()                                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(bufs, idx, wt, out)
        for a, b in zip(ref, got):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"


def test_packed_and_epilogue_graph(dev):
    w = W.WORKLOADS["dsr1_decode"]
    o = OracleRun.get(w)
    say("[graph] packed layout + fused epilogue")
    logits = torch.from_numpy(o.logits).to(dev)
    x = W.make_x(w).to(dev)
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device=dev)
    wt = torch.empty(w.T, w.k, dtype=torch.float32, device=dev)
    bufs = moe.PackedBuffers.allocate(w.T, w.H, w.E, w.k, w.fp8, dev)
    y = torch.randn(w.T * w.k, w.H, device=dev).to(torch.bfloat16)
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    gamma = torch.rand(w.H, device=dev).to(torch.bfloat16)
    res_out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    step = moe.PreparedStep(logits, w.k, x, w.C, w.fp8, bufs, y, out, idx, wt, stream=side,
                            route_groups=(8, 4), epilogue=(x, gamma, 1e-6, res_out))
    for t in (idx, wt, bufs.token_slot, bufs.recv_src, bufs.expert_offsets, out, res_out):
        t.zero_()
    torch.cuda.synchronize()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.route_and_dispatch()
        step.combine()
    side.synchronize()
    ref = _outputs(bufs, idx, wt, out, (bufs.expert_offsets, res_out))
    # against the oracle: grouped routing, packed slots, combine + residual + RMSNorm
    idx_o, w_o = oracle.route_topk_grouped(o.logits, w.k, 8, 4)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    np.testing.assert_allclose(wt.cpu().numpy(), w_o, rtol=W_RTOL, atol=0)
    offs_o, pslot_o, _ = oracle.assign_packed(idx_o, w.E)
    np.testing.assert_array_equal(bufs.expert_offsets.cpu().numpy(), offs_o)
    np.testing.assert_array_equal(bufs.token_slot.cpu().numpy(), pslot_o)
    y_pairs = dev_bits(y)[pslot_o.reshape(-1)]
    res_o, normed_o = oracle.combine_residual_rmsnorm(y_pairs, pslot_o, wt.cpu().numpy(), W.bits(x.cpu()),
                                                      dev_bits(gamma), 1e-6)
    assert (dev_bits(res_out) == res_o).all()
    assert (dev_bits(out) == normed_o).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step.route_and_dispatch()
        step.combine()
    for rep in range(4):
        for t in (idx, wt, bufs.token_slot, bufs.recv_src, bufs.expert_offsets, out, res_out):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(bufs, idx, wt, out, (bufs.expert_offsets, res_out))
        for a, b in zip(ref, got):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"
