"""Pins for the oracle's packed, count-sized dispatch layout (handbook
"NVSHMEM and DeepEP", "High-throughput mode": counts per destination first,
then a receive buffer of exactly that size; pplx blog, Dispatch: tokens
contiguous per expert).

Independent checks: numpy's bincount/cumsum for the offsets, numpy's stable
argsort of the flattened expert ids for the row order, a per-pair brute
force count, and the relation to the fixed-slot oracle (pinned on its own).
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _ids(rng, T, E, k):
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("name", W.ORDER)
def test_offsets_and_order_match_numpy(name):
    w = W.WORKLOADS[name]
    idx, _ = oracle.route_topk(W.make_logits(w).numpy(), w.k)
    offsets, slot, src = oracle.assign_packed(idx, w.E)
    flat = idx.reshape(-1)
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=w.E))]))
    order = np.argsort(flat, kind="stable")          # pairs sorted by expert, then by pair index
    np.testing.assert_array_equal(slot.reshape(-1)[order], np.arange(w.T * w.k))
    np.testing.assert_array_equal(src, order // w.k)


@pytest.mark.parametrize("name", ["tiny", "mixtral_prefill", "dsr1_decode", "glm_prefill"])
def test_relation_to_fixed_slots(name):
    """With C = T nothing is dropped and packed row = offsets[e] + (fixed slot - e*C)."""
    w = W.WORKLOADS[name]
    idx, _ = oracle.route_topk(W.make_logits(w).numpy(), w.k)
    offsets, slot, src = oracle.assign_packed(idx, w.E)
    counts, fslot, fsrc = oracle.assign_slots(idx, w.E, w.T)
    np.testing.assert_array_equal(slot, offsets[idx] + (fslot - idx * w.T))
    np.testing.assert_array_equal(np.diff(offsets), counts)


def test_brute_force_rows():
    rng = np.random.default_rng(4)
    for T, E, k in ((1, 1, 1), (5, 3, 2), (9, 6, 3), (17, 8, 8), (30, 5, 1)):
        idx = _ids(rng, T, E, k)
        offsets, slot, src = oracle.assign_packed(idx, E)
        for t in range(T):
            for j in range(k):
                e = idx[t, j]
                row = int((idx < e).sum()) + int((idx[:t] == e).sum())
                assert slot[t, j] == row
                assert src[row] == t
        assert offsets[E] == T * k


def test_dense_rows_are_the_packed_layout():
    """The oracle's dense filled-row listing (ascending slot order) is the
    packed buffer: row p holds x of recv_src[p]."""
    w = W.WORKLOADS["tiny"]
    idx, _ = oracle.route_topk(W.make_logits(w).numpy(), w.k)
    x = W.bits(W.make_x(w))
    counts, _, fsrc = oracle.assign_slots(idx, w.E, w.C)
    rows, _, _ = oracle.pack(x, oracle.BF16, fsrc, counts, w.C)
    _, _, src = oracle.assign_packed(idx, w.E)
    np.testing.assert_array_equal(rows, x[src])


def test_empty_and_rejects_bad_ids():
    offsets, slot, src = oracle.assign_packed(np.zeros((0, 2), np.int32), 4)
    assert (offsets == 0).all() and slot.shape == (0, 2) and src.size == 0
    with pytest.raises(Exception):
        oracle.assign_packed(np.array([[0, 4]], np.int32), 4)
