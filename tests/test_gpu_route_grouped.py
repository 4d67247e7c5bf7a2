"""GPU parity of the group-limited ("node-limited") router
(handbook "NVSHMEM and DeepEP", "High-throughput mode": score each node by
the sum of its two best expert scores, keep the best nodes, pick the top
experts among them), through the C ABI, against the CPU oracle.

Ids must be identical; weights within the router tolerance.  Cases: the
DeepSeek-R1 and GLM expert counts at full token counts, the handbook's worked
example, group layouts on both kernel paths (whole power-of-two lane runs per
group, and groups that split lanes or span odd lane counts), planted ties
between group scores and between logits, signed zeros, equal rows, ragged
token counts, and the reduction to the plain router when every group is kept.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
import oracle
import workloads as W
from gpu_common import W_RTOL, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _check(dev, logits, k, G, M, label):
    say(f"[grouped route] {label}: T={logits.shape[0]} E={logits.shape[1]} k={k} groups={G} kept={M}")
    idx_g, w_g = moe.moe_route_topk_grouped(torch.from_numpy(logits).to(dev), k, G, M)
    idx_o, w_o = oracle.route_topk_grouped(logits, k, G, M)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w_g.cpu().numpy(), w_o, rtol=W_RTOL, atol=0)
    return idx_o


@pytest.mark.parametrize("name,G,M", [("dsr1_decode", 8, 4), ("dsr1_prefill", 8, 4), ("glm_prefill", 8, 4),
                                      ("glm_prefill", 16, 3), ("mixtral_prefill", 4, 2)])
def test_workload_logits(dev, name, G, M):
    w = W.WORKLOADS[name]
    logits = W.make_logits(w).numpy()
    idx = _check(dev, logits, w.k, G, M, name)
    gs = w.E // G
    assert max(len(set(r)) for r in (idx // gs).tolist()) <= M


def test_page_worked_example(dev):
    rng = np.random.default_rng(0)
    scores = rng.random((4096, 256)) + rng.random(256) * 0.5
    _check(dev, scores.astype(np.float32), 8, 8, 4, "handbook example")


def _rows(rng, T, E):
    rows = rng.standard_normal((T, E)).astype(np.float32)
    kind = np.arange(T) % 5
    rows[kind == 1] = rng.integers(-2, 3, (int((kind == 1).sum()), E)).astype(np.float32)
    rows[kind == 2] = rng.choice(np.array([0.0, -0.0, 0.5, -0.5], np.float32), (int((kind == 2).sum()), E))
    rows[kind == 3] = np.float32(-1.5)
    return rows


# (E, G, M, k): lanes per group = E/G/VPL with VPL = 1, 2, 4, 8, 16 for E <= 64, 128, 256, 512, 1024
CASES = [
    (8, 4, 2, 2), (8, 2, 1, 3), (16, 8, 3, 4), (40, 5, 2, 6), (48, 3, 2, 8), (64, 2, 1, 16), (64, 1, 1, 5),
    (12, 4, 2, 3), (60, 6, 4, 7),                      # groups that are not a power-of-two run of lanes
    (96, 8, 3, 8), (128, 8, 4, 8), (100, 10, 4, 8),     # VPL 2: aligned, aligned, split lanes
    (192, 6, 3, 8), (256, 8, 4, 8), (256, 64, 8, 8), (256, 16, 1, 16), (200, 8, 2, 9),
    (512, 16, 4, 16), (384, 8, 2, 8),
    (1024, 64, 6, 16), (1024, 8, 4, 8), (600, 8, 3, 12), (1024, 2, 1, 16),
]


@pytest.mark.parametrize("E,G,M,k", CASES)
@pytest.mark.parametrize("many", [False, True])
def test_group_layouts(dev, E, G, M, k, many):
    """Both kernel layouts: one token per wave, and (from 6144 tokens, at
    most 16 groups) four tokens per wave; ragged token counts."""
    rng = np.random.default_rng(31 * E + 7 * G + 3 * M + k + many)
    T = (6200 if many else 1000) + (E % 7)
    _check(dev, _rows(rng, T, E), k, G, M, "layout")


@pytest.mark.parametrize("E,G,k", [(256, 8, 8), (128, 4, 8), (60, 6, 4), (8, 4, 2)])
def test_all_groups_kept_equals_plain_route(dev, E, G, k):
    rng = np.random.default_rng(E + G + k)
    logits = torch.from_numpy(_rows(rng, 777, E)).to(dev)
    a_idx, a_w = moe.moe_route_topk_grouped(logits, k, G, G)
    b_idx, b_w = moe.moe_route_topk(logits, k)
    assert torch.equal(a_idx, b_idx)
    np.testing.assert_allclose(a_w.cpu().numpy(), b_w.cpu().numpy(), rtol=W_RTOL, atol=0)


def test_equal_group_scores_take_the_lower_group(dev):
    """Every group has the same two best logits: the kept groups must be
    0 .. M-1, and the experts the lowest-index maxima inside them."""
    E, G, M, k = 256, 8, 4, 8
    rng = np.random.default_rng(3)
    rows = rng.uniform(-1, 0.5, (64, E)).astype(np.float32)
    rows.reshape(64, G, E // G)[:, :, 5] = 2.0
    rows.reshape(64, G, E // G)[:, :, 9] = 1.0
    idx = _check(dev, rows, k, G, M, "equal group scores")
    assert set((idx // (E // G)).reshape(-1).tolist()) == {0, 1, 2, 3}


def test_empty_and_single_token(dev):
    z = torch.empty(0, 256, dtype=torch.float32, device=dev)
    i, w = moe.moe_route_topk_grouped(z, 8, 8, 4)
    assert i.shape == (0, 8)
    rng = np.random.default_rng(1)
    _check(dev, rng.standard_normal((1, 256)).astype(np.float32), 8, 8, 4, "one token")
