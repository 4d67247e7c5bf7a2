"""Pins for the oracle's combine epilogue: residual add and RMSNorm
("How GPUs Talk to Each Other During LLM Inference", section 5: right after
the sum, add the residual stream, store it, and apply the next module's
RMSNorm, x * rsqrt(mean of squares + eps) * gamma).

Independent checks: torch's bf16 conversion for the residual output,
torch.nn.functional.rms_norm in float64 for the normalised output (the
oracle must be its nearest bf16 value), closed forms (a constant row
normalises to sign * gamma; scaling a row by a power of two changes nothing
when eps = 0; one element), and the one-step double -> bf16 rounding on
values where rounding through float first would differ.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _bf16(a):
    return W.bits(torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16))


def _f(bits):
    return W.from_bits(np.ascontiguousarray(bits, np.uint16)).float().numpy()


def _case(rng, T, H, k, drop=0.0):
    slot = np.arange(T * k, dtype=np.int32).reshape(T, k)
    slot[rng.random((T, k)) < drop] = -1
    w = rng.random((T, k)).astype(np.float32)
    y = _bf16(rng.standard_normal((T * k, H)))
    res = _bf16(rng.standard_normal((T, H)) * 2)
    gamma = _bf16(rng.uniform(0.5, 1.5, H))
    return y, slot, w, res, gamma


def test_residual_out_single_expert_matches_torch():
    rng = np.random.default_rng(1)
    T, H = 64, 96
    y, slot, _, res, gamma = _case(rng, T, H, 1)
    w = np.ones((T, 1), np.float32)
    res_out, _ = oracle.combine_residual_rmsnorm(y, slot, w, res, gamma, 1e-6)
    want = (W.from_bits(y).float() + W.from_bits(res).float()).to(torch.bfloat16)
    np.testing.assert_array_equal(res_out, W.bits(want))


def test_residual_out_is_the_rounded_sum_plus_residual():
    rng = np.random.default_rng(2)
    T, H, k = 50, 128, 8
    y, slot, w, res, gamma = _case(rng, T, H, k, drop=0.2)
    res_out, _ = oracle.combine_residual_rmsnorm(y, slot, w, res, gamma, 1e-6)
    _, acc = oracle.combine(y, slot, w, want_acc=True)
    r = (acc + _f(res)).astype(np.float32)
    np.testing.assert_array_equal(res_out, _bf16(r))


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-5, 0.5])
def test_normed_is_nearest_bf16_of_torch_rms_norm(eps):
    rng = np.random.default_rng(3)
    T, H, k = 40, 256, 4
    y, slot, w, res, gamma = _case(rng, T, H, k, drop=0.1)
    _, normed = oracle.combine_residual_rmsnorm(y, slot, w, res, gamma, eps)
    _, acc = oracle.combine(y, slot, w, want_acc=True)
    r = torch.from_numpy((acc + _f(res)).astype(np.float32)).double()
    exact = torch.nn.functional.rms_norm(r, (H,), weight=torch.from_numpy(_f(gamma)).double(), eps=eps).numpy()
    got = _f(normed).astype(np.float64)
    # the two bf16 neighbours around the exact value: got must be the nearer
    ulp = np.ldexp(1.0, np.frexp(np.abs(got))[1] - 8)
    assert (np.abs(got - exact) <= 0.5 * ulp * (1 + 1e-9) + 1e-300).all()


def test_constant_row_normalises_to_gamma():
    T, H = 6, 64
    rng = np.random.default_rng(4)
    gamma = _bf16(rng.uniform(0.25, 2, H))
    vals = np.array([3.0, -0.75, 1e-3, -1e3, 2.0 ** -100, 7.0], np.float32)
    res = _bf16(np.repeat(vals[:, None], H, axis=1))
    y = np.zeros((T, H), np.uint16)
    slot = np.full((T, 1), -1, np.int32)            # nothing routed: r = residual
    _, normed = oracle.combine_residual_rmsnorm(y, slot, np.zeros((T, 1), np.float32), res, gamma, 0.0)
    want = np.where(vals[:, None] < 0, -_f(gamma)[None, :], _f(gamma)[None, :])
    np.testing.assert_array_equal(_f(normed), want)


def test_power_of_two_scaling_is_invisible_without_eps():
    rng = np.random.default_rng(5)
    T, H = 8, 128
    base = rng.standard_normal((T, H)).astype(np.float32)
    gamma = _bf16(rng.uniform(0.5, 1.5, H))
    slot = np.full((T, 1), -1, np.int32)
    y = np.zeros((T, H), np.uint16)
    w = np.zeros((T, 1), np.float32)
    outs = [oracle.combine_residual_rmsnorm(y, slot, w, _bf16(base * 2.0 ** s), gamma, 0.0)[1] for s in (-20, 0, 9)]
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[1], outs[2])


def test_one_element_rows():
    vals = np.array([2.0, -3.0, 0.5, 0.0], np.float32)
    eps = 0.25
    res = _bf16(vals[:, None])
    gamma = _bf16(np.array([1.5], np.float32))
    slot = np.full((4, 1), -1, np.int32)
    _, normed = oracle.combine_residual_rmsnorm(np.zeros((4, 1), np.uint16), slot, np.zeros((4, 1), np.float32),
                                                res, gamma, eps)
    exact = vals / np.sqrt(vals.astype(np.float64) ** 2 + eps) * 1.5
    np.testing.assert_array_equal(normed.reshape(-1), oracle.bf16_round_double_array(exact))
    np.testing.assert_allclose(_f(normed).reshape(-1), exact, rtol=2 ** -8)


def test_double_rounding_is_one_step():
    # 1 + 2^-8 is the midpoint between bf16 1.0 and 1 + 2^-7; a double just
    # above it rounds up, although rounding it to float first gives the
    # midpoint, which would then go to the even neighbour 1.0
    v = np.array([1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -40),
                  2.0 ** -130, 3 * 2.0 ** -134, 3.5e38, 0.0, -0.0], np.float64)
    got = oracle.bf16_round_double_array(v)
    want = [0x3F81, 0x3F80, 0x3F82, 0xBF81, 0x0008, 0x0000 | 0x0002, 0x7F80, 0x0000, 0x8000]
    assert [int(g) for g in got] == want
    # on values a float holds exactly it agrees with the float rounding
    f = np.random.default_rng(6).standard_normal(10000).astype(np.float32)
    np.testing.assert_array_equal(oracle.bf16_round_double_array(f.astype(np.float64)), oracle.bf16_round_array(f))


def test_rejects_bad_eps():
    with pytest.raises(Exception):
        oracle.combine_residual_rmsnorm(np.zeros((1, 8), np.uint16), np.zeros((1, 1), np.int32),
                                        np.ones((1, 1), np.float32), np.zeros((1, 8), np.uint16),
                                        np.zeros(8, np.uint16), -1.0)


def test_normed_is_rounded_once_from_the_exact_value():
    """Over a million elements, the normalised output equals the one-step bf16
    rounding of torch's float64 RMSNorm, except where that value lies within
    1e-12 (relative) of a rounding midpoint.  Rounding through float first
    would differ on the ~1 in 2^16 values near a midpoint."""
    rng = np.random.default_rng(8)
    T, H, k = 1024, 1024, 2
    y, slot, w, res, gamma = _case(rng, T, H, k)
    _, normed = oracle.combine_residual_rmsnorm(y, slot, w, res, gamma, 1e-6)
    _, acc = oracle.combine(y, slot, w, want_acc=True)
    r = torch.from_numpy((acc + _f(res)).astype(np.float32)).double()
    exact = torch.nn.functional.rms_norm(r, (H,), weight=torch.from_numpy(_f(gamma)).double(), eps=1e-6).numpy()
    want = oracle.bf16_round_double_array(exact)
    diff = normed != want
    if diff.any():
        e = exact[diff]
        m, ex = np.frexp(np.abs(e))
        frac = np.ldexp(m, 8) - np.floor(np.ldexp(m, 8))      # position between two bf16 neighbours
        assert (np.abs(frac - 0.5) < 1e-12 * 256).all(), "a value away from a midpoint rounded differently"
