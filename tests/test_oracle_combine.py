"""Pins for the oracle's combine: out[t] = bf16(sum_j w[t,j] * y[t,j]) with
float32 fused multiply-adds in top-k order (pplx blog, Combine: the weighted
sum of the experts' unquantised 16-bit outputs is formed at the receiver into
a caller-allocated tensor; "How GPUs Talk", section 7: the k weighted outputs
are added up at the token's origin).

Checked against exact rational arithmetic with the float32 accumulation
error bound, against torch's bf16 rounding, and on special cases whose
result is known exactly.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _bf16_value(b: int) -> float:
    return float(np.array([b << 16], np.uint32).view(np.float32)[0])


def _bf16_ulp(v: float) -> float:
    if v == 0:
        return 2.0 ** -133
    e = np.frexp(abs(v))[1] - 1
    return 2.0 ** (max(e, -126) - 7)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-38).astype(np.float32),          # subnormals
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.3895314e38, 3.4028235e38,
                  np.inf, -np.inf, 0.0, -0.0, 1e-45], np.float32),
    ])
    # exact ties: random bf16 values plus half a bf16 ulp
    base = (rng.integers(0, 0x7F00, 50_000).astype(np.uint32) << 16)
    vals = np.concatenate([vals, (base | 0x8000).view(np.float32), (base | 0x7FFF).view(np.float32)])
    mine = oracle.bf16_round_array(vals)
    lib = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, lib)
    nan = oracle.bf16_round(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


@pytest.mark.parametrize("seed", range(3))
def test_combine_within_exact_rational_bound(seed):
    rng = np.random.default_rng(seed)
    T, k, H = 24, 5, 16
    y = W.bits(torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).to(torch.bfloat16))
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    slot = np.arange(T * k, dtype=np.int32).reshape(T, k)
    slot[rng.uniform(size=(T, k)) < 0.15] = -1
    out, acc = oracle.combine(y, slot, w, want_acc=True)
    for t in range(T):
        for h in range(H):
            terms = [Fraction(float(w[t, j])) * Fraction(_bf16_value(int(y[t * k + j, h])))
                     for j in range(k) if slot[t, j] >= 0]
            exact = sum(terms, Fraction(0))
            mag = sum((abs(x) for x in terms), Fraction(0))
            # each fused multiply-add rounds once, to at most half an ulp of a
            # partial sum bounded by the sum of magnitudes
            bound = Fraction(k) * Fraction(2) ** -24 * mag
            assert abs(Fraction(float(acc[t, h])) - exact) <= bound
            # the final bf16 rounding is correctly rounded from acc
            a = float(acc[t, h])
            got = _bf16_value(int(out[t, h]))
            assert abs(got - a) <= _bf16_ulp(a) / 2


def test_accumulation_order_and_precision():
    # y0 = 1, y1 = 1.5 * 2^-24, y2 = -1, all weights 1:
    # fp32 in order j=0,1,2 gives (1 + 2^-23) - 1 = 2^-23 exactly;
    # exact arithmetic would give 1.5 * 2^-24, reverse order a different value.
    vals = np.array([1.0, 1.5 * 2 ** -24, -1.0], np.float32)
    y = W.bits(torch.from_numpy(vals).to(torch.bfloat16)).reshape(3, 1)
    out, acc = oracle.combine(y, np.array([[0, 1, 2]], np.int32), np.ones((1, 3), np.float32), want_acc=True)
    assert acc[0, 0] == np.float32(2.0 ** -23)
    assert _bf16_value(int(out[0, 0])) == 2.0 ** -23


def test_fused_multiply_add_single_rounding():
    # w = 1 + 2^-23, y = 1 + 2^-7 (bf16), acc starts at -1 (j = 0 term).  The
    # product 1 + 2^-7 + 2^-23 + 2^-30 needs 31 bits: a float multiply drops
    # the 2^-30 term, a fused multiply-add keeps it (the result fits 24 bits).
    w = np.array([[1.0, 1 + 2.0 ** -23]], np.float32)
    vals = np.array([-1.0, 1 + 2.0 ** -7], np.float32)
    y = W.bits(torch.from_numpy(vals).to(torch.bfloat16)).reshape(2, 1)
    _, acc = oracle.combine(y, np.array([[0, 1]], np.int32), w, want_acc=True)
    assert acc[0, 0] == np.float32(2.0 ** -7 + 2.0 ** -23 + 2.0 ** -30)
    assert np.float32(2.0 ** -7 + 2.0 ** -23 + 2.0 ** -30) != np.float32(2.0 ** -7 + 2.0 ** -23)


def test_k1_unit_weight_returns_row():
    rng = np.random.default_rng(4)
    y = W.bits(torch.from_numpy(rng.standard_normal((50, 64)).astype(np.float32)).to(torch.bfloat16))
    out = oracle.combine(y, np.arange(50, dtype=np.int32).reshape(50, 1), np.ones((50, 1), np.float32))
    np.testing.assert_array_equal(out, y)


def test_one_hot_weights_select_row():
    rng = np.random.default_rng(5)
    T, k, H = 16, 4, 32
    y = W.bits(torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).to(torch.bfloat16))
    pick = rng.integers(0, k, T)
    w = np.zeros((T, k), np.float32)
    w[np.arange(T), pick] = 1.0
    out = oracle.combine(y, np.arange(T * k, dtype=np.int32).reshape(T, k), w)
    want = y[np.arange(T) * k + pick]
    # +0 accumulators stay +0 where the picked value is -0: compare values
    np.testing.assert_array_equal(out.view(np.int16).astype(np.int32) & 0x7FFF, want.astype(np.int32) & 0x7FFF)


def test_all_dropped_gives_positive_zero():
    y = np.full((2, 8), 0x3F80, np.uint16)
    out = oracle.combine(y, np.array([[-1, -1]], np.int32), np.ones((1, 2), np.float32))
    assert (out == 0).all()


@pytest.mark.parametrize("name", ["tiny", "mixtral_prefill", "dsr1_decode"])
def test_identity_experts_scale_input_by_weight_sum(name):
    w = W.WORKLOADS[name]
    idx, wt = oracle.route_topk(W.make_logits(w).numpy(), w.k)
    counts, token_slot, recv_src = oracle.assign_slots(idx, w.E, w.C)
    x = W.bits(W.make_x(w))
    y_pairs = np.repeat(x, w.k, axis=0)                 # every expert returns its input
    out, acc = oracle.combine(y_pairs, token_slot, wt, want_acc=True)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sw = wt.astype(np.float64).sum(axis=1, keepdims=True)
    want = sw * xf
    bound = w.k * 2.0 ** -24 * np.abs(want) + 1e-45
    assert np.all(np.abs(acc - want) <= bound)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - want) <= ulp / 2 + bound)
