"""Pins for the oracle's group-limited ("node-limited") router
(handbook "NVSHMEM and DeepEP", "High-throughput mode": each node is scored
by the sum of its two best expert scores, only the best nodes stay eligible,
and the top experts are picked among them).

Independent checks: the figures the handbook prints for its worked example
(4096 seeded tokens over 8 nodes of 32 experts; the measures are recomputed
here from their definitions), a brute force that characterises the kept groups
and the chosen experts by pairwise dominance instead of repeated selection,
and special cases that reduce to the plain router (pinned on its own) or to
closed forms.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "node_limited_routing.json")


def _membership(unit_of_choice: np.ndarray, n_units: int) -> np.ndarray:
    """Boolean [T, n_units]: True where at least one of the token's chosen
    experts lies in that unit (an expert, a GPU or a node)."""
    T = unit_of_choice.shape[0]
    m = np.zeros((T, n_units), dtype=bool)
    m[np.repeat(np.arange(T), unit_of_choice.shape[1]), unit_of_choice.reshape(-1)] = True
    return m


def _traffic_measures(idx: np.ndarray, spec: dict) -> dict:
    """The worked example's per-token means, for a source GPU on node 0.  A
    copy leaves the node once per distinct destination at the level that
    deduplicates: per chosen expert, per GPU or per node.  Units are numbered
    so that node 0 holds the first ones at every level; the source node's own
    units send nothing over the network."""
    T = idx.shape[0]
    n_gpus = spec["nodes"] * spec["gpus_per_node"]
    experts_per_gpu = spec["experts"] // n_gpus
    levels = {"expert": (1, spec["experts"]), "gpu": (experts_per_gpu, n_gpus),
              "node": (experts_per_gpu * spec["gpus_per_node"], spec["nodes"])}
    local = {"expert": experts_per_gpu * spec["gpus_per_node"], "gpu": spec["gpus_per_node"], "node": 1}
    out = {}
    for level, (experts_per_unit, n_units) in levels.items():
        hit = _membership(idx // experts_per_unit, n_units)
        if level == "node":
            out["nodes_touched"] = hit.sum(axis=1).mean()
        copies = hit[:, local[level]:].sum(axis=1).mean()
        out[f"copies_per_{level}"] = copies
        # NIC time of the batch: bytes sent over the network / NIC bandwidth
        out[f"ms_per_{level}"] = T * copies * spec["token_bytes"] / spec["nic_bytes_per_s"] * 1e3
    return out


def _page_scores(spec: dict) -> np.ndarray:
    """The seeded router scores of the worked example, from the draw the
    golden file records (float64 draws, then float32 for the routers)."""
    d = spec["draw"]
    assert d["generator"] == "numpy.random.default_rng"
    stream = np.random.default_rng(d["seed"])
    per_pair = stream.random(spec["tokens"] * spec["experts"]).reshape(spec["tokens"], spec["experts"])
    per_expert = stream.random(spec["experts"])
    return (per_pair + d["expert_offset_scale"] * per_expert[None, :]).astype(np.float32)


def test_page_worked_example():
    spec = json.load(open(GOLDEN))
    logits = _page_scores(spec)
    k, G, M = spec["topk"], spec["nodes"], spec["max_nodes"]
    free_idx, _ = oracle.route_topk(logits, k)
    lim_idx, _ = oracle.route_topk_grouped(logits, k, G, M)
    for name, idx in (("unlimited", free_idx), ("limited", lim_idx)):
        got = _traffic_measures(idx, spec)
        for key, printed in spec["printed"][name].items():
            assert round(got[key], 2) == pytest.approx(printed, abs=1e-9), (name, key, got[key], printed)
    # every token stays within M nodes under the limit
    experts_per_node = spec["experts"] // G
    assert _membership(lim_idx // experts_per_node, G).sum(axis=1).max() <= M


def _scores(row, G):
    gs = len(row) // G
    out = []
    for g in range(G):
        grp = row[g * gs:(g + 1) * gs]
        # the largest fp32 sum over all pairs of distinct members
        out.append(max(np.float32(grp[a]) + np.float32(grp[b]) for a, b in itertools.combinations(range(gs), 2)))
    return out


def _beats(va, ia, vb, ib):
    return va > vb or (va == vb and ia < ib)


def _brute(row, k, G, M):
    """Kept groups: the unique M-subset each of whose members beats every
    group outside it (score, then lower index).  Chosen experts: the unique
    k-subset of eligible experts each of whose members beats every other
    eligible expert (logit, then lower index), listed in that order."""
    E = len(row)
    gs = E // G
    sc = _scores(row, G)
    kept = [s for s in itertools.combinations(range(G), M)
            if all(_beats(sc[g], g, sc[h], h) for g in s for h in range(G) if h not in s)]
    assert len(kept) == 1
    elig = [e for e in range(E) if e // gs in kept[0]]
    chosen = [s for s in itertools.combinations(elig, k)
              if all(_beats(row[a], a, row[b], b) for a in s for b in elig if b not in s)]
    assert len(chosen) == 1
    order = sorted(chosen[0], key=lambda e: (-float(row[e]), e))
    return order


def _rows(rng, n, E):
    rows = rng.standard_normal((n, E)).astype(np.float32)
    for i in range(n):
        kind = i % 4
        if kind == 1:
            rows[i] = rng.integers(-2, 3, E).astype(np.float32)     # many ties, equal group scores
        elif kind == 2:
            rows[i] = rng.choice(np.array([0.0, -0.0, 0.5, -0.5], np.float32), E)
        elif kind == 3:
            rows[i] = np.float32(1.25)
    return rows


@pytest.mark.parametrize("E,G,M,k", [(4, 2, 1, 1), (6, 3, 1, 2), (6, 3, 2, 3), (8, 4, 2, 2), (8, 4, 2, 4),
                                     (8, 2, 1, 3), (9, 3, 2, 4), (12, 4, 3, 5), (12, 6, 2, 4), (10, 5, 5, 3)])
def test_matches_brute_force(E, G, M, k):
    rng = np.random.default_rng(7 * E + 3 * G + M + k)
    rows = _rows(rng, 48, E)
    idx, _ = oracle.route_topk_grouped(rows, k, G, M)
    for t in range(rows.shape[0]):
        assert list(idx[t]) == _brute(rows[t], k, G, M), (t, rows[t])


def test_all_groups_kept_is_plain_topk():
    rng = np.random.default_rng(5)
    for E, G, k in ((8, 4, 2), (64, 8, 6), (256, 8, 8), (128, 16, 8)):
        rows = _rows(rng, 200, E)
        a_idx, a_w = oracle.route_topk_grouped(rows, k, G, G)
        b_idx, b_w = oracle.route_topk(rows, k)
        np.testing.assert_array_equal(a_idx, b_idx)
        np.testing.assert_array_equal(a_w, b_w)


def test_weights_are_the_full_softmax():
    """Limiting the groups changes the choice, not the distribution: each
    weight equals the plain router's full-softmax weight of that expert."""
    w = W.WORKLOADS["dsr1_decode"]
    logits = W.make_logits(w).numpy()
    idx, wt = oracle.route_topk_grouped(logits, w.k, 8, 4)
    _, w_all = oracle.route_topk(logits, w.E)          # k = E: every expert's weight, in rank order
    i_all, _ = oracle.route_topk(logits, w.E)
    full = np.empty_like(w_all)
    np.put_along_axis(full, i_all, w_all, axis=1)
    np.testing.assert_array_equal(wt, np.take_along_axis(full, idx, axis=1))


def test_pair_groups_closed_form():
    """Groups of two: a group's score is the sum of both members."""
    rng = np.random.default_rng(9)
    rows = rng.standard_normal((300, 16)).astype(np.float32)
    idx, _ = oracle.route_topk_grouped(rows, 4, 8, 2)
    for t in range(rows.shape[0]):
        sc = rows[t, 0::2] + rows[t, 1::2]
        order = sorted(range(8), key=lambda g: (-float(sc[g]), g))
        kept = set(order[:2])
        assert sorted(idx[t]) == sorted(e for g in kept for e in (2 * g, 2 * g + 1))


def test_whole_groups_when_k_fills_them():
    """k = M * group size: the chosen experts are exactly the M best groups."""
    rng = np.random.default_rng(11)
    rows = rng.standard_normal((300, 32)).astype(np.float32)
    G, M = 8, 3
    idx, _ = oracle.route_topk_grouped(rows, M * 4, G, M)
    for t in range(rows.shape[0]):
        groups = sorted(set(int(e) // 4 for e in idx[t]))
        assert len(groups) == M
        top2 = np.sort(rows[t].reshape(G, 4), axis=1)[:, -2:]
        sc = top2[:, 0] + top2[:, 1]
        out = [g for g in range(G) if g not in groups]
        assert min(sc[groups]) >= max(sc[out])


def test_rejects_bad_group_arguments():
    x = np.zeros((2, 8), np.float32)
    for k, G, M in ((2, 3, 1), (2, 8, 1), (2, 4, 0), (2, 4, 5), (5, 4, 2)):
        with pytest.raises(Exception):
            oracle.route_topk_grouped(x, k, G, M)
