"""Pins for the oracle's dispatch steps: per-expert counts, fixed-slot
assignment in ascending token order, and the bf16 row pack.

Checked against numpy's bincount and stable argsort (a stable sort by
expert is the "sort by destination" step of the handbook's EP flow, section
"Why MoE's all-to-all is hard"), brute-force ranks on tiny inputs, and the
invariants a fixed-slot receive buffer must satisfy (handbook, "Low-latency
mode"; pplx blog, Dispatch: contiguous per-expert buffers plus each token's
source index).
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _route(name):
    w = W.WORKLOADS[name]
    idx, _ = oracle.route_topk(W.make_logits(w).numpy(), w.k)
    return w, idx


@pytest.mark.parametrize("name", W.ORDER)
def test_counts_match_bincount(name):
    w, idx = _route(name)
    counts, _, _ = oracle.assign_slots(idx, w.E, w.C)
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=w.E))
    assert counts.sum() == w.T * w.k


@pytest.mark.parametrize("name", W.ORDER)
def test_slots_match_stable_sort(name):
    w, idx = _route(name)
    counts, token_slot, recv_src = oracle.assign_slots(idx, w.E, w.C)
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")          # (t, j) pairs grouped by expert
    starts = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=w.E))])
    want_slot = np.empty(flat.size, np.int64)
    for e in range(w.E):
        pairs = order[starts[e]:starts[e + 1]]
        r = np.arange(pairs.size)
        assert pairs.size <= w.C                     # these workloads never overflow
        want_slot[pairs] = e * w.C + r
        np.testing.assert_array_equal(recv_src[e * w.C: e * w.C + pairs.size], pairs // w.k)
        assert (recv_src[e * w.C + pairs.size:(e + 1) * w.C] == -1).all()
    np.testing.assert_array_equal(token_slot.ravel(), want_slot)


@pytest.mark.parametrize("name", W.ORDER)
def test_slot_invariants(name):
    w, idx = _route(name)
    counts, token_slot, recv_src = oracle.assign_slots(idx, w.E, w.C)
    filled = recv_src >= 0
    # every token appears exactly k times
    np.testing.assert_array_equal(np.bincount(recv_src[filled], minlength=w.T), np.full(w.T, w.k))
    # round trip: the slot of (t, j) holds t, and sits in expert idx[t, j]'s range
    t_of = np.repeat(np.arange(w.T), w.k)
    np.testing.assert_array_equal(recv_src[token_slot.ravel()], t_of)
    np.testing.assert_array_equal(token_slot.ravel() // w.C, idx.ravel())
    # strictly ascending sources within each expert
    for e in range(w.E):
        seg = recv_src[e * w.C: e * w.C + counts[e]]
        assert (np.diff(seg) > 0).all()


def test_ranks_brute_force_tiny():
    rng = np.random.default_rng(21)
    for trial in range(20):
        E = int(rng.integers(1, 12))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(0, 30))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32).reshape(T, k)
        C = int(rng.integers(1, T + 2))
        counts, token_slot, recv_src = oracle.assign_slots(idx, E, C)
        for t in range(T):
            for j in range(k):
                e = idx[t, j]
                r = sum(1 for t2 in range(t) if e in idx[t2])
                assert token_slot[t, j] == (e * C + r if r < C else -1)
                if r < C:
                    assert recv_src[e * C + r] == t
        for e in range(E):
            assert counts[e] == (idx == e).sum()


def test_overflow_drops_later_tokens():
    # every token picks expert 0 first: capacity 5 keeps tokens 0..4 only
    T, E, k, C = 12, 4, 2, 5
    idx = np.array([[0, 1 + (t % 3)] for t in range(T)], np.int32)
    counts, token_slot, recv_src = oracle.assign_slots(idx, E, C)
    assert counts[0] == T                       # true count, above capacity
    assert (token_slot[:C, 0] == np.arange(C)).all()
    assert (token_slot[C:, 0] == -1).all()
    np.testing.assert_array_equal(recv_src[:C], np.arange(C))
    for e in (1, 2, 3):
        assert counts[e] == 4 and (token_slot[:, 1][idx[:, 1] == e] >= 0).all()


def test_rejects_bad_expert_id():
    with pytest.raises(ValueError):
        oracle.assign_slots(np.array([[0, 9]], np.int32), 4, 2)


@pytest.mark.parametrize("name", ["tiny", "mixtral_prefill", "dsr1_prefill"])
def test_pack_bf16_is_row_copy(name):
    w, idx = _route(name)
    counts, token_slot, recv_src = oracle.assign_slots(idx, w.E, w.C)
    x = W.bits(W.make_x(w))
    rows, scales, slot_of_row = oracle.pack(x, oracle.BF16, recv_src, counts, w.C)
    assert scales is None and rows.shape == (w.T * w.k, w.H)
    assert (np.diff(slot_of_row) > 0).all()
    np.testing.assert_array_equal(rows, x[recv_src[slot_of_row]])
    # the slot of (t, j) holds x[t]
    pos = np.searchsorted(slot_of_row, token_slot.ravel())
    np.testing.assert_array_equal(rows[pos], np.repeat(x, w.k, axis=0))


def test_pack_empty_batch():
    counts, token_slot, recv_src = oracle.assign_slots(np.zeros((0, 2), np.int32), 8, 4)
    assert (counts == 0).all() and (recv_src == -1).all()
    rows, _, slot_of_row = oracle.pack(np.zeros((0, 128), np.uint16), oracle.BF16, recv_src, counts, 4)
    assert rows.shape == (0, 128) and slot_of_row.shape == (0,)
