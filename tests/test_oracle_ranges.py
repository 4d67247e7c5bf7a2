"""The oracle's range forms (used by the benchmark's host-cores baseline to
run the oracle's own C functions on disjoint token or expert ranges in
threads) give exactly what the whole-array calls give.  Marshalling only:
no arithmetic of the method is involved in the split."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import bench
import oracle
import workloads as W


def _sample(name, T):
    w = W.WORKLOADS[name]
    ws = w.with_(T=T, C=T)
    logits = np.ascontiguousarray(W.make_logits(w)[:T].numpy())
    x = np.ascontiguousarray(W.bits(W.make_x(w)[:T]))
    y = np.ascontiguousarray(W.bits(W.make_y_pairs(w, rows=T * w.k)))
    return ws, logits, x, y


@pytest.mark.parametrize("name,T,parts", [("mixtral_prefill", 300, 7), ("dsr1_decode", 128, 5),
                                          ("glm_prefill", 96, 16), ("tiny", 64, 3)])
def test_threaded_ranges_equal_whole_calls(name, T, parts):
    ws, logits, x, y = _sample(name, T)
    dtype = oracle.FP8_E4M3 if ws.fp8 else oracle.BF16
    idx, wt = oracle.route_topk(logits, ws.k)
    counts, slot, src = oracle.assign_slots(idx, ws.E, ws.C)
    rows, scales, slot_of_row = oracle.pack(x, dtype, src, counts, ws.C)
    out = oracle.combine(y, slot, wt)

    bounds = [(T * i // parts, T * (i + 1) // parts) for i in range(parts)]
    with ThreadPoolExecutor(parts) as pool:
        idx2 = np.empty_like(idx)
        wt2 = np.empty_like(wt)
        list(pool.map(lambda b: oracle.route_topk_range(logits, ws.k, idx2, wt2, *b), bounds))
        np.testing.assert_array_equal(idx2, idx)
        np.testing.assert_array_equal(wt2.view(np.uint32), wt.view(np.uint32))

        filled = np.minimum(counts, ws.C)
        ranges = bench._balanced_expert_ranges(filled, parts)
        assert ranges[0][0] == 0 and ranges[-1][1] == ws.E
        assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))
        rows2 = np.empty_like(rows)
        scales2 = None if scales is None else np.empty_like(scales)
        sor2 = np.empty_like(slot_of_row)
        list(pool.map(lambda r: oracle.pack_range(x, dtype, src, counts, ws.C, rows2, scales2, sor2, *r), ranges))
        for e0, e1, p0 in ranges:
            n = int(filled[e0:e1].sum())
            sor2[p0:p0 + n] += e0 * ws.C          # range slots are relative to the range's first expert
        np.testing.assert_array_equal(sor2, slot_of_row)
        np.testing.assert_array_equal(rows2, rows)
        if scales is not None:
            np.testing.assert_array_equal(scales2.view(np.uint32), scales.view(np.uint32))

        out2 = np.empty_like(out)
        list(pool.map(lambda b: oracle.combine_range(y, slot, wt, out2, *b), bounds))
        np.testing.assert_array_equal(out2, out)

        gamma = np.ascontiguousarray(x[0])
        res_o, normed_o = oracle.combine_residual_rmsnorm(y, slot, wt, x, gamma, 1e-6)
        res2, normed2 = np.empty_like(res_o), np.empty_like(normed_o)
        list(pool.map(lambda b: oracle.combine_residual_rmsnorm_range(y, slot, wt, x, gamma, 1e-6, res2, normed2, *b),
                      bounds))
        np.testing.assert_array_equal(res2, res_o)
        np.testing.assert_array_equal(normed2, normed_o)

        if ws.H % 128 == 0:
            q, sc = oracle.quantize_rows_fp8(normed_o)
            q2, sc2 = np.empty_like(q), np.empty_like(sc)
            list(pool.map(lambda b: oracle.quantize_rows_fp8_range(normed_o, q2, sc2, *b), bounds))
            np.testing.assert_array_equal(q2, q)
            np.testing.assert_array_equal(sc2.view(np.uint32), sc.view(np.uint32))


def test_balanced_ranges_cover_every_expert_once():
    rng = np.random.default_rng(3)
    for _ in range(50):
        E = int(rng.integers(1, 300))
        filled = rng.integers(0, 50, E) * (rng.random(E) < 0.7)
        parts = int(rng.integers(1, 20))
        r = bench._balanced_expert_ranges(filled, parts)
        assert 1 <= len(r) <= parts
        assert r[0][0] == 0 and r[-1][1] == E
        for (a0, a1, p0), (b0, b1, q0) in zip(r, r[1:]):
            assert a1 == b0 and q0 == p0 + int(filled[a0:a1].sum())
