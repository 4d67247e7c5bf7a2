"""The benchmark's copy floors (bench_floor.hip) move the bytes they are
compared against: floor_scatter_rows writes every filled slot's row (the
whole bf16 row, or H code bytes plus one 4-byte word per 128 elements) and
nothing else; floor_gather_rows reads each token's k slotted rows and writes
one row per token; floor_scatter_writes stores what floor_scatter_rows stores,
at the same slots, without reading the source.  Checked on small dispatches
through the library, so the slot maps are the real ones."""
import numpy as np
import pytest
import torch

import bench
import combine_moe_route_amd as moe
from gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu

SENT = 0x5A


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("T,H,E,k,fp8", [(300, 256, 16, 4, False), (300, 512, 16, 4, True), (1000, 1024, 8, 2, False),
                                         (200, 384, 64, 8, True)])
def test_floor_kernels_touch_exactly_the_slotted_rows(dev, T, H, E, k, fp8):
    say(f"[floor] T={T} H={H} E={E} k={k} fp8={fp8}")
    lib = bench.floor_lib()
    g = torch.Generator(device="cpu")
    g.manual_seed(T + H + E)
    logits = torch.randn(T, E, generator=g).to(dev)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).to(dev)
    C = T
    idx, wt, bufs = moe.moe_route_dispatch(logits, x, k, C, fp8=fp8)
    slots = bufs.token_slot.cpu().numpy()
    # scatter into fresh, sentinel-filled rows
    rows = torch.full((E * C, H * (1 if fp8 else 2)), SENT, dtype=torch.uint8, device=dev)
    scales = torch.full((E * C, H // 128 * 4), SENT, dtype=torch.uint8, device=dev) if fp8 else None
    s = torch.cuda.current_stream().cuda_stream
    rc = lib.floor_scatter_rows(x.data_ptr(), T, H, int(fp8), bufs.token_slot.data_ptr(), k, rows.data_ptr(),
                                scales.data_ptr() if fp8 else None, s)
    assert rc == 0
    torch.cuda.synchronize()
    filled = np.zeros(E * C, bool)
    filled[slots[slots >= 0]] = True
    r = rows.cpu().numpy()
    xb = x.view(torch.uint8).cpu().numpy().reshape(T, 2 * H)
    assert (r[~filled] == SENT).all(), "a row outside the slots was written"
    for t in range(T):
        for j in range(k):
            sl = slots[t, j]
            if not fp8:
                np.testing.assert_array_equal(r[sl], xb[t])          # the row itself
            else:
                lo_hi = xb[t].reshape(-1, 2, 16)                     # per 16-element group: two 16 B halves
                np.testing.assert_array_equal(r[sl], np.bitwise_xor(lo_hi[:, 0], lo_hi[:, 1]).reshape(-1))
    if fp8:
        sc = scales.cpu().numpy()
        assert (sc[~filled] == SENT).all()
        assert (sc[filled] != SENT).any()
    # gather: every token's row written, from the rows its slots name
    y = torch.randint(0, 256, (E * C, 2 * H), dtype=torch.uint8, device=dev)
    out = torch.full((T, 2 * H), SENT, dtype=torch.uint8, device=dev)
    rc = lib.floor_gather_rows(y.data_ptr(), E * C, H, bufs.token_slot.data_ptr(), wt.data_ptr(), T, k,
                               out.data_ptr(), s)
    assert rc == 0
    torch.cuda.synchronize()
    yh = y.cpu().numpy().view(np.uint32).reshape(E * C, -1, 4)
    oh = out.cpu().numpy().view(np.uint32).reshape(T, -1, 4)
    wb = wt.cpu().numpy().view(np.uint32)
    for t in range(T):
        want = np.zeros_like(oh[t])
        want[:, 0] = np.bitwise_xor.reduce(wb[t])
        for j in range(k):
            want ^= yh[slots[t, j]]
        np.testing.assert_array_equal(oh[t], want)


@pytest.mark.parametrize("T,H,E,k,fp8", [(300, 256, 16, 4, False), (300, 512, 16, 4, True), (1000, 1024, 8, 2, False),
                                         (200, 384, 64, 8, True)])
def test_floor_writes_touch_exactly_the_slotted_rows(dev, T, H, E, k, fp8):
    """floor_scatter_writes stores every filled slot's whole row (and scale
    words) with the copy's pattern made from (token, vector), and nothing
    outside the slots."""
    say(f"[floor writes] T={T} H={H} E={E} k={k} fp8={fp8}")
    lib = bench.floor_lib()
    g = torch.Generator(device="cpu")
    g.manual_seed(T * 3 + H + E)
    logits = torch.randn(T, E, generator=g).to(dev)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).to(dev)
    C = T
    _, _, bufs = moe.moe_route_dispatch(logits, x, k, C, fp8=fp8)
    slots = bufs.token_slot.cpu().numpy()
    rows = torch.full((E * C, H * (1 if fp8 else 2)), SENT, dtype=torch.uint8, device=dev)
    scales = torch.full((E * C, H // 128 * 4), SENT, dtype=torch.uint8, device=dev) if fp8 else None
    rc = lib.floor_scatter_writes(T, H, int(fp8), bufs.token_slot.data_ptr(), k, rows.data_ptr(),
                                  scales.data_ptr() if fp8 else None, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    filled = np.zeros(E * C, bool)
    filled[slots[slots >= 0]] = True
    r = rows.cpu().numpy()
    assert (r[~filled] == SENT).all(), "a row outside the slots was written"
    nvec = r.shape[1] // 16
    v = np.arange(nvec, dtype=np.uint32)
    for t in range(T):
        tt = np.full(nvec, t, np.uint32)
        want = np.stack([tt, v, ~tt, ~v], axis=1).reshape(-1).view(np.uint8)
        for j in range(k):
            np.testing.assert_array_equal(r[slots[t, j]], want)
    if fp8:
        sc = scales.cpu().numpy().view(np.uint32)
        assert (scales.cpu().numpy()[~filled] == SENT).all()
        for t in range(T):
            for j in range(k):
                np.testing.assert_array_equal(sc[slots[t, j]], np.full(H // 128, t, np.uint32))


def test_placement_probe_runs(dev):
    """bench.py --placement times the same dispatch into separately allocated
    buffers and prints one JSON object with every figure filled in."""
    import json
    import os
    import subprocess
    import sys
    say("[placement probe] tiny, 2 buffers")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--workload", "tiny", "--placement", "2"],
                       cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    p = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1])["placement"]
    assert p["workload"] == "tiny" and len(p["receive_buffers"]) == 2 and len(p["expert_output_buffers"]) == 1
    for b in p["receive_buffers"]:
        assert len(b["dispatch_us"]) == 2 and min(b["dispatch_us"]) > 0 and b["sequential_fill_tbps"] > 0
    assert all(v > 0 for v in p["capacity_sweep_first_buffer_us"].values())
    assert min(p["expert_output_buffers"][0]["combine_us"]) > 0
