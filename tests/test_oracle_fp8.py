"""Pins for the oracle's fp8 dispatch encoding: OCP E4M3 codes with one fp32
scale per 128 elements (handbook "NVSHMEM and DeepEP", section
"High-throughput mode": FP8 for dispatch with fine-grained scaling, one scale
per 128 elements; the traffic listing sizes the row as hidden bytes plus one
fp32 per 128).

The E4M3 format itself is the OCP 8-bit floating point specification (OFP8,
E4M3: bias 7, max normal 448, subnormal step 2^-9, S.1111.111 is NaN, no
infinities).  The oracle's encoder is pinned against an independent decoder,
against torch's float8_e4m3fn conversion (a library routine, which rounds to
nearest-even but turns values past the rounding range into NaN, so it is
compared only below 464), exhaustively over all bf16 inputs, and by the
quantisation error bound.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _decode(code: int) -> float:
    """E4M3 value of a code, written from the format definition."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# anchor values of the OFP8 E4M3 table
ANCHORS = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
           0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0}


def test_decoder_anchors_and_library():
    for c, v in ANCHORS.items():
        assert _decode(c) == v
    assert math.isnan(_decode(0x7F)) and math.isnan(_decode(0xFF))
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mine = np.array([_decode(c) for c in range(256)], np.float32)
    np.testing.assert_array_equal(np.isnan(lib), np.isnan(mine))
    ok = ~np.isnan(mine)
    np.testing.assert_array_equal(lib[ok], mine[ok])


def test_encode_roundtrip_all_codes():
    for c in range(256):
        v = _decode(c)
        if math.isnan(v):
            continue
        assert oracle.e4m3_encode(v) == c, hex(c)


def test_midpoints_round_to_even():
    pos = sorted({_decode(c) for c in range(0x7F)})          # 0 .. 448
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = (lo + hi) / 2                                     # exact in float32
        c_lo, c_hi = oracle.e4m3_encode(lo), oracle.e4m3_encode(hi)
        even = c_lo if c_lo % 2 == 0 else c_hi
        assert oracle.e4m3_encode(mid) == even, (lo, hi)
        assert oracle.e4m3_encode(-mid) == even | 0x80
        below = np.nextafter(np.float32(mid), np.float32(0))
        above = np.nextafter(np.float32(mid), np.float32(1000))
        assert oracle.e4m3_encode(float(below)) == c_lo
        assert oracle.e4m3_encode(float(above)) == c_hi


def test_saturation_nan_and_signed_zero():
    for v in (448.0, 449.0, 463.99, 464.0, 500.0, 1e30, math.inf):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    assert oracle.e4m3_encode(math.nan) & 0x7F == 0x7F
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80


def test_matches_torch_on_all_bf16_in_range():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (allbits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) < 464.0)
    vals = vals[keep]
    mine = oracle.e4m3_encode_array(vals)
    lib = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, lib)


def test_matches_torch_on_random_float32():
    rng = np.random.default_rng(2024)
    mag = np.exp2(rng.uniform(-14, math.log2(463.9), 400_000))
    vals = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    mine = oracle.e4m3_encode_array(vals)
    lib = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, lib)


def _dequant(codes, scales):
    dec = np.array([_decode(c) for c in range(256)], np.float64)
    return dec[codes].reshape(-1, 128) * scales.astype(np.float64)[:, None]


@pytest.mark.parametrize("seed", range(4))
def test_quantize_row_error_bound_and_amax(seed):
    rng = np.random.default_rng(seed)
    H = 1024
    x = torch.from_numpy(rng.standard_normal(H).astype(np.float32) * 10 ** rng.uniform(-3, 3, H)
                         .astype(np.float32)).to(torch.bfloat16)
    xb = W.bits(x)
    codes, scales = oracle.quantize_row_fp8(xb)
    xf = x.float().numpy().astype(np.float64).reshape(-1, 128)
    amax = np.abs(xf).max(axis=1)
    # the scale maps the block's largest magnitude onto 448 (to fp32 rounding)
    np.testing.assert_allclose(scales * 448.0, amax, rtol=2.0 ** -23)
    # the largest element of each block encodes to +-448
    for b in range(H // 128):
        i = int(np.argmax(np.abs(xf[b])))
        assert codes[b * 128 + i] & 0x7F == 0x7E
    err = np.abs(xf - _dequant(codes, scales))
    ratio = np.abs(xf) / scales[:, None].astype(np.float64)
    normal = ratio >= 2.0 ** -6
    rel_tol = 2.0 ** -4 * (1 + 2.0 ** -20)
    assert np.all(err[normal] <= rel_tol * np.abs(xf[normal]))
    sub_tol = 2.0 ** -10 * (1 + 2.0 ** -20) * np.broadcast_to(scales[:, None], xf.shape)
    assert np.all(err[~normal] <= sub_tol[~normal])


def test_zero_block_scale_one_and_blocks_independent():
    x = np.zeros(384, np.uint16)
    x[256:] = W.bits(torch.full((128,), -3.0, dtype=torch.bfloat16))
    x[5] = 0x8000                                    # -0.0 in a zero block
    codes, scales = oracle.quantize_row_fp8(x)
    assert scales[0] == 1.0 and scales[1] == 1.0
    assert codes[5] == 0x80 and (np.delete(codes[:256], 5) == 0).all()
    assert (codes[256:] == 0xFE).all()
    np.testing.assert_allclose(scales[2], 3.0 / 448.0, rtol=2.0 ** -23)


def test_quantize_rejects_ragged_hidden():
    with pytest.raises(ValueError):
        oracle.quantize_row_fp8(np.zeros(200, np.uint16))


@pytest.mark.parametrize("name", ["dsr1_decode"])
def test_pack_fp8_rows_are_quantised_sources(name):
    w = W.WORKLOADS[name]
    idx, _ = oracle.route_topk(W.make_logits(w).numpy(), w.k)
    counts, token_slot, recv_src = oracle.assign_slots(idx, w.E, w.C)
    x = W.bits(W.make_x(w))
    rows, scales, slot_of_row = oracle.pack(x, oracle.FP8_E4M3, recv_src, counts, w.C)
    assert rows.dtype == np.uint8 and scales.shape == (w.T * w.k, w.H // 128)
    per_token = [oracle.quantize_row_fp8(x[t]) for t in range(w.T)]
    for p, s in enumerate(slot_of_row):
        t = recv_src[s]
        np.testing.assert_array_equal(rows[p], per_token[t][0])
        np.testing.assert_array_equal(scales[p], per_token[t][1])


def _rows_with_edge_blocks(n: int, H: int, seed: int) -> np.ndarray:
    """Seeded bf16 rows [n, H] of widely spread magnitudes, with an all-zero
    block, a block holding the largest finite bf16 magnitude and a block of
    tiny (subnormal-code) values in some rows."""
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-4, 4, (n, H))
    x = torch.from_numpy((rng.standard_normal((n, H)) * mag).astype(np.float32)).to(torch.bfloat16)
    xb = W.bits(x).reshape(n, H).copy()
    nblk = H // 128
    for r in range(n):
        b = r % nblk
        if r % 3 == 0:
            xb[r, b * 128:(b + 1) * 128] = 0                       # all-zero block: scale 1
        elif r % 3 == 1:
            xb[r, b * 128 + (r % 128)] = 0x7F7F                    # largest finite bf16
            xb[r, b * 128 + ((r + 1) % 128)] = 0xFF7F              # and its negative
        else:
            xb[r, b * 128:(b + 1) * 128] = 0x0001                  # smallest bf16 subnormal
    return xb


@pytest.mark.parametrize("n,H", [(0, 128), (1, 128), (3, 6144), (257, 128), (5, 7168), (4, 6144)])
def test_quantize_rows_equals_row_by_row(n, H):
    """The batch form must give, row for row, what the per-row encoding
    (pinned above by the E4M3 table, torch's conversion and the error bound)
    gives: one scale per 128 elements of the same row, codes at the same
    positions.  A wrong code or scale stride, or a row offset, shows here."""
    xb = _rows_with_edge_blocks(n, H, seed=n * 31 + H)
    codes, scales = oracle.quantize_rows_fp8(xb)
    assert codes.shape == (n, H) and scales.shape == (n, H // 128)
    for r in range(n):
        c1, s1 = oracle.quantize_row_fp8(xb[r])
        np.testing.assert_array_equal(codes[r], c1, err_msg=f"row {r} codes")
        np.testing.assert_array_equal(scales[r], s1, err_msg=f"row {r} scales")


def test_quantize_rows_edge_blocks_decode_within_bound():
    """Independent of the per-row function: every block of the batch form
    dequantises to its own source block within the E4M3 error bound, the
    zero blocks get scale 1, and the largest finite bf16 magnitude maps onto
    448 exactly (the block's amax code)."""
    n, H = 6, 384
    xb = _rows_with_edge_blocks(n, H, seed=7)
    codes, scales = oracle.quantize_rows_fp8(xb)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    deq = _dequant(codes.reshape(-1), scales.reshape(-1)).reshape(n, H)
    sc = np.repeat(scales.astype(np.float64), 128, axis=1)
    ratio = np.abs(xf) / sc
    normal = ratio >= 2.0 ** -6
    err = np.abs(xf - deq)
    assert np.all(err[normal] <= 2.0 ** -4 * (1 + 2.0 ** -20) * np.abs(xf[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * (1 + 2.0 ** -20) * sc[~normal])
    for r in range(n):
        b = r % (H // 128)
        blk = slice(b * 128, (b + 1) * 128)
        if r % 3 == 0:
            assert scales[r, b] == 1.0 and (codes[r, blk] == 0).all()
        elif r % 3 == 1:
            assert codes[r, b * 128 + (r % 128)] == 0x7E
            assert codes[r, b * 128 + ((r + 1) % 128)] == 0xFE
            np.testing.assert_allclose(scales[r, b] * 448.0, float(np.float32(xf[r, b * 128 + (r % 128)])),
                                       rtol=2.0 ** -23)


def test_quantize_rows_agrees_with_pack_on_decode_workload():
    """The rows the GPU tests take their expected codes from must be those
    oracle.pack writes into the slots (same workload, same sources)."""
    w = W.WORKLOADS["dsr1_decode"]
    idx, _ = oracle.route_topk(W.make_logits(w).numpy(), w.k)
    counts, _, recv_src = oracle.assign_slots(idx, w.E, w.C)
    x = W.bits(W.make_x(w))
    rows, scales, slot_of_row = oracle.pack(x, oracle.FP8_E4M3, recv_src, counts, w.C)
    codes, blk_scales = oracle.quantize_rows_fp8(x)
    src = recv_src[slot_of_row]
    np.testing.assert_array_equal(rows, codes[src])
    np.testing.assert_array_equal(scales, blk_scales[src])
