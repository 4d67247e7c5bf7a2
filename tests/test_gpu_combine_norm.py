"""GPU parity of the fused combine epilogue (moe_combine_residual_rmsnorm;
"How GPUs Talk to Each Other During LLM Inference", section 5: residual add
and RMSNorm right after the sum) through the C ABI, against the CPU oracle.

residual_out must be bit-identical (the same fp32 operations in the same
order as the oracle: combine's fma chain, one fp32 add, nearest-even bf16).
normed_out within one bf16 ulp: both sides evaluate the norm in double and
round once, but the kernel adds the squares in its own order, so an element
can land on the other side of a rounding midpoint.  The fp8 output's codes
and scales must equal the oracle's encoding of the oracle's own normalised
rows in every 128-element block whose bf16 values match bit for bit (and the
encoding of the kernel's own bf16 rows everywhere).  Cases: the five
workloads at full size (fixed slots), the packed layout, in-place residual
update, dropped pairs, row widths on every vector-count path, k from 1 to
16, eps = 0 with constant rows, a batch long enough to take several
launches, and canaries past the outputs.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_amd as moe
import oracle
import workloads as W
from gpu_common import OracleRun, bf16_ulp_distance, dev_bits, place_rows, require_gpu, say, to_dev_bf16

pytestmark = pytest.mark.gpu

SENT_BF16 = 0x7FBD


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _bf16(a):
    return W.bits(torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16))


def _compare(label, res_g, normed_g, res_o, normed_o):
    np.testing.assert_array_equal(res_g, res_o)
    d = bf16_ulp_distance(normed_g, normed_o)
    say(f"  {label}: normed max ulp {int(d.max(initial=0))}, not identical {int((d > 0).sum())} of {d.size}")
    assert d.max(initial=0) <= 1


def _run(dev, y_dev, slot, w, res_bits, gamma_bits, eps, in_place=False):
    T, H = res_bits.shape
    res = to_dev_bf16(res_bits, dev)
    gamma = to_dev_bf16(gamma_bits, dev)
    normed = torch.empty(T + 1, H, dtype=torch.bfloat16, device=dev)
    normed.view(torch.int16).fill_(SENT_BF16)
    res_out = res if in_place else torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    moe.moe_combine_residual_rmsnorm(y_dev, torch.from_numpy(slot).to(dev), torch.from_numpy(w).to(dev), res, gamma,
                                     eps, residual_out=res_out, normed_out=normed[:T])
    got = dev_bits(normed)
    assert (got[T] == SENT_BF16).all(), "normed_out written past its end"
    return dev_bits(res_out), got[:T]


@pytest.mark.parametrize("name", W.ORDER)
def test_workloads_full_size(dev, name):
    w = W.WORKLOADS[name]
    o = OracleRun.get(w)
    say(f"[combine+norm] {name}")
    rng = np.random.default_rng(w.seed)
    res_bits = _bf16(rng.standard_normal((w.T, w.H)))
    gamma_bits = _bf16(rng.uniform(0.5, 1.5, w.H))
    y = place_rows(w, o.y_pairs, o.token_slot, dev)
    res_g, normed_g = _run(dev, y, o.token_slot, o.wt, res_bits, gamma_bits, 1e-6)
    res_o, normed_o = oracle.combine_residual_rmsnorm(o.y_pairs, o.token_slot, o.wt, res_bits, gamma_bits, 1e-6)
    _compare(name, res_g, normed_g, res_o, normed_o)
    del y


def test_packed_layout_in_place(dev):
    w = W.WORKLOADS["dsr1_decode"]
    o = OracleRun.get(w)
    offsets, slot, _ = oracle.assign_packed(o.idx, w.E)
    rng = np.random.default_rng(5)
    res_bits = _bf16(rng.standard_normal((w.T, w.H)) * 4)
    gamma_bits = _bf16(rng.uniform(-1, 1, w.H))
    y = torch.empty(w.T * w.k, w.H, dtype=torch.bfloat16, device=dev)
    y.index_copy_(0, torch.from_numpy(slot.reshape(-1).astype(np.int64)).to(dev), to_dev_bf16(o.y_pairs, dev))
    res_g, normed_g = _run(dev, y, slot, o.wt, res_bits, gamma_bits, 1e-5, in_place=True)
    res_o, normed_o = oracle.combine_residual_rmsnorm(o.y_pairs, slot, o.wt, res_bits, gamma_bits, 1e-5)
    _compare("packed, in place", res_g, normed_g, res_o, normed_o)


@pytest.mark.parametrize("T,H,k", [(1, 8, 1), (3, 64, 2), (50, 2048, 3), (37, 2056, 8), (20, 4104, 4),
                                   (64, 7168, 8), (9, 16384, 16), (17, 8192, 5), (300, 1024, 16), (129, 6144, 2),
                                   # 512 tokens and more: 256-thread groups with 1, 2 and 8 vectors per lane,
                                   # and 512-thread groups with 2 (rows of 4097 to 8192 elements)
                                   (600, 1024, 3), (700, 4096, 2), (520, 6152, 8), (513, 8192, 4), (512, 9000, 4)])
def test_shapes(dev, T, H, k):
    rng = np.random.default_rng(T * 7 + H + k)
    rows = T * k
    slot = rng.permutation(rows).astype(np.int32).reshape(T, k)
    slot[rng.random((T, k)) < 0.15] = -1                       # dropped pairs are skipped
    past = rng.random((T, k)) < 0.02                           # so are slots at or past E*C
    slot[past] = rows + rng.integers(0, 1 << 20, int(past.sum()))
    wt = rng.random((T, k)).astype(np.float32)
    y_rows = _bf16(rng.standard_normal((rows, H)))
    y_pairs = np.zeros((rows, H), np.uint16)
    keep = (slot.reshape(-1) >= 0) & (slot.reshape(-1) < rows)
    y_pairs[keep] = y_rows[slot.reshape(-1)[keep]]
    res_bits = _bf16(rng.standard_normal((T, H)) * rng.choice([1e-3, 1.0, 50.0], (T, 1)))
    gamma_bits = _bf16(rng.uniform(0.25, 2.0, H))
    say(f"[combine+norm] T={T} H={H} k={k}")
    res_g, normed_g = _run(dev, to_dev_bf16(y_rows, dev).view(1, rows, H), slot, wt, res_bits, gamma_bits, 1e-6)
    kept = np.where(keep.reshape(T, k), slot, -1).astype(np.int32)
    res_o, normed_o = oracle.combine_residual_rmsnorm(y_pairs, kept, wt, res_bits, gamma_bits, 1e-6)
    _compare(f"T={T} H={H} k={k}", res_g, normed_g, res_o, normed_o)


def test_constant_rows_without_eps(dev):
    """Nothing routed, eps = 0: each row is its residual, a constant c, and
    normalises to sign(c) * gamma exactly on both sides."""
    T, H = 6, 512
    vals = np.array([3.0, -0.75, 1e-3, -1e3, 2.0 ** -100, 7.0], np.float32)
    res_bits = _bf16(np.repeat(vals[:, None], H, axis=1))
    gamma_bits = _bf16(np.random.default_rng(6).uniform(0.25, 2, H))
    slot = np.full((T, 2), -1, np.int32)
    wt = np.zeros((T, 2), np.float32)
    y = torch.zeros(1, 8, H, dtype=torch.bfloat16, device=dev)
    res_g, normed_g = _run(dev, y, slot, wt, res_bits, gamma_bits, 0.0)
    res_o, normed_o = oracle.combine_residual_rmsnorm(np.zeros((T * 2, H), np.uint16), slot, wt, res_bits,
                                                      gamma_bits, 0.0)
    np.testing.assert_array_equal(res_g, res_o)
    np.testing.assert_array_equal(normed_g, normed_o)


def test_empty(dev):
    y = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device=dev)
    e = torch.empty(0, 2, dtype=torch.int32, device=dev)
    r, n = moe.moe_combine_residual_rmsnorm(y, e, torch.empty(0, 2, device=dev),
                                            torch.empty(0, 64, dtype=torch.bfloat16, device=dev),
                                            torch.ones(64, dtype=torch.bfloat16, device=dev))
    assert r.shape == (0, 64) and n.shape == (0, 64)


def test_batch_longer_than_one_launch(dev):
    """One work-group per token and at most 2^32 - 1 work-items per launch:
    a batch of more than 2^22 tokens is run as several launches.  The tokens
    on both sides of the piece boundary, the first and last ones and a random
    sample are checked against the oracle; every row is checked for being
    written."""
    piece = 1 << 22
    T, H, k = piece + 300, 8, 2
    rng = np.random.default_rng(22)
    slot = np.arange(T * k, dtype=np.int32).reshape(T, k)
    slot[rng.random((T, k)) < 0.1] = -1
    wt = rng.random((T, k), dtype=np.float32)
    y_bits = _bf16(rng.standard_normal((T * k, H), dtype=np.float32))
    res_bits = _bf16(rng.standard_normal((T, H), dtype=np.float32))
    gamma_bits = _bf16(rng.uniform(0.5, 1.5, H))
    say(f"[combine+norm] T={T} (two launches) H={H} k={k}")
    res_g, normed_g = _run(dev, to_dev_bf16(y_bits, dev).view(1, T * k, H), slot, wt, res_bits, gamma_bits, 1e-6)
    assert not (normed_g == SENT_BF16).all(axis=1).any()
    picks = np.unique(np.concatenate([np.arange(0, 64), np.arange(piece - 200, T), rng.integers(0, T, 2000)]))
    y_pairs = np.where((slot.reshape(-1) >= 0)[:, None], y_bits, 0).astype(np.uint16).reshape(T, k, H)
    res_o, normed_o = oracle.combine_residual_rmsnorm(y_pairs[picks].reshape(-1, H), slot[picks], wt[picks],
                                                      res_bits[picks], gamma_bits, 1e-6)
    _compare(f"T={T}, {picks.size} sampled tokens", res_g[picks], normed_g[picks], res_o, normed_o)


# ---- fp8 re-quantisation of the normalised rows (moe_combine_residual_rmsnorm_fp8) ----
#
# The codes are a function of the kernel's own bf16 normalised values, so
# they are compared bit for bit with the oracle's E4M3 block encoding of
# those values (the float decides the integer in one precision on both
# sides); the bf16 values themselves are held to the one-ulp bar above.

def _run_fp8(dev, y_dev, slot, w, res_bits, gamma_bits, eps, keep_bf16):
    T, H = res_bits.shape
    res = to_dev_bf16(res_bits, dev)
    gamma = to_dev_bf16(gamma_bits, dev)
    q = torch.full(((T + 1) * H + 64,), 0xA5, dtype=torch.uint8, device=dev)
    sc = torch.full(((T + 1) * (H // 128) + 16,), -7.0, dtype=torch.float32, device=dev)
    res_out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    normed = torch.empty(T, H, dtype=torch.bfloat16, device=dev) if keep_bf16 else None
    T_ = torch.from_numpy(slot).to(dev)
    W_ = torch.from_numpy(w).to(dev)
    if y_dev.dim() == 2:
        y_dev = y_dev.view(1, y_dev.shape[0], H)
    E, C, _ = y_dev.shape
    lib = moe.load()
    rc = lib.moe_combine_residual_rmsnorm_fp8(y_dev.data_ptr(), E, C, H, T_.data_ptr(), W_.data_ptr(), T,
                                              slot.shape[1], res.data_ptr(), gamma.data_ptr(), float(eps),
                                              res_out.data_ptr(), normed.data_ptr() if keep_bf16 else None,
                                              q.data_ptr(), sc.data_ptr(), None)
    assert rc == 0, moe.moe_status_string(rc)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    sch = sc.cpu().numpy()
    assert (qh[T * H:] == 0xA5).all(), "codes written past their end"
    assert (sch[T * (H // 128):] == -7.0).all(), "scales written past their end"
    return (dev_bits(res_out), dev_bits(normed) if keep_bf16 else None, qh[:T * H].reshape(T, H),
            sch[:T * (H // 128)].reshape(T, H // 128))


def _check_fp8(label, dev, y_dev, slot, w, y_pairs, res_bits, gamma_bits, eps, slot_o=None):
    """slot_o: the oracle's view of the slots (out-of-range ones as -1), if it differs."""
    res_g, normed_g, q_g, sc_g = _run_fp8(dev, y_dev, slot, w, res_bits, gamma_bits, eps, True)
    res_o, normed_o = oracle.combine_residual_rmsnorm(y_pairs, slot if slot_o is None else slot_o, w, res_bits,
                                                      gamma_bits, eps)
    _compare(label, res_g, normed_g, res_o, normed_o)
    # end to end: the codes and scales of the oracle's own normalised rows.
    # Every 128-element block whose bf16 values equal the oracle's bit for
    # bit must encode identically; a block may differ only where a value of
    # it sits one ulp off (the kernel sums the squares in its own order).
    T, H = normed_o.shape
    q_e, sc_e = oracle.quantize_rows_fp8(normed_o)
    same_vals = (normed_g.reshape(T, H // 128, 128) == normed_o.reshape(T, H // 128, 128)).all(axis=2)
    same_enc = (q_g.reshape(T, H // 128, 128) == q_e.reshape(T, H // 128, 128)).all(axis=2) & \
        (sc_g.view(np.uint32) == sc_e.view(np.uint32))
    assert same_enc[same_vals].all(), f"{label}: a block with identical bf16 values encodes differently"
    say(f"  {label}: fp8 blocks differing from the oracle's own rows {int((~same_enc).sum())}, "
        f"blocks holding a 1-ulp value {int((~same_vals).sum())} of {same_vals.size}")
    assert (~same_enc).sum() <= (~same_vals).sum()
    # and bit for bit the encoding of the kernel's own bf16 rows
    q_o, sc_o = oracle.quantize_rows_fp8(normed_g)
    np.testing.assert_array_equal(q_g, q_o)
    np.testing.assert_array_equal(sc_g.view(np.uint32), sc_o.view(np.uint32))
    # without the bf16 rows: the same codes, scales and residual
    res_2, _, q_2, sc_2 = _run_fp8(dev, y_dev, slot, w, res_bits, gamma_bits, eps, False)
    np.testing.assert_array_equal(res_2, res_g)
    np.testing.assert_array_equal(q_2, q_g)
    np.testing.assert_array_equal(sc_2.view(np.uint32), sc_g.view(np.uint32))


@pytest.mark.parametrize("name", W.ORDER)
def test_fp8_output_workloads(dev, name):
    w = W.WORKLOADS[name]
    o = OracleRun.get(w)
    say(f"[combine+norm fp8] {name}")
    rng = np.random.default_rng(w.seed + 1)
    res_bits = _bf16(rng.standard_normal((w.T, w.H)))
    gamma_bits = _bf16(rng.uniform(0.5, 1.5, w.H))
    y = place_rows(w, o.y_pairs, o.token_slot, dev)
    _check_fp8(name, dev, y, o.token_slot, o.wt, o.y_pairs, res_bits, gamma_bits, 1e-6)
    del y


@pytest.mark.parametrize("T,H,k", [(1, 128, 1), (5, 256, 2), (300, 2048, 8), (513, 1024, 3), (40, 7168, 16),
                                   (600, 16384, 2), (77, 6144, 5), (640, 4096, 2), (520, 6144, 8)])
def test_fp8_output_shapes(dev, T, H, k):
    rng = np.random.default_rng(T * 5 + H + k)
    rows = T * k
    slot = rng.permutation(rows).astype(np.int32).reshape(T, k)
    slot[rng.random((T, k)) < 0.15] = -1
    wt = rng.random((T, k)).astype(np.float32)
    y_rows = _bf16(rng.standard_normal((rows, H)))
    y_pairs = np.zeros((rows, H), np.uint16)
    keep = slot.reshape(-1) >= 0
    y_pairs[keep] = y_rows[slot.reshape(-1)[keep]]
    # row scales from tiny to large, a zero block and a block with one spike
    res_bits = _bf16(rng.standard_normal((T, H)) * rng.choice([1e-30, 1e-3, 1.0, 300.0], (T, 1)))
    gamma_bits = _bf16(rng.uniform(0.25, 2.0, H))
    gamma_bits[:128] = 0                                        # block 0 normalises to all zeros
    gamma_bits[200 % H] = _bf16(np.array([1e4]))[0] if H > 256 else gamma_bits[200 % H]
    say(f"[combine+norm fp8] T={T} H={H} k={k}")
    _check_fp8(f"fp8 T={T} H={H} k={k}", dev, to_dev_bf16(y_rows, dev), slot, wt, y_pairs, res_bits, gamma_bits,
               1e-6)


@pytest.mark.parametrize("seed", range(40))
def test_random_shapes(dev, seed):
    """Seeded random shapes through both epilogue entry points: T from 1 to
    3000 (both sides of the 512-token switch), H up to the largest supported
    (a multiple of 128 for the fp8 output), k from 1 to 16, eps from 0 to
    1e-2, dropped and out-of-range slots, rows of very different scales."""
    rng = np.random.default_rng(90_000 + seed)
    fp8 = bool(seed % 2)
    T = int(rng.choice([rng.integers(1, 512), rng.integers(512, 3001)]))
    H = 128 * int(rng.integers(1, 129)) if fp8 else 8 * int(rng.integers(1, 2049))
    k = int(rng.integers(1, 17))
    eps = float(rng.choice([0.0, 1e-6, 1e-2]))
    rows = T * k
    slot = rng.permutation(rows).astype(np.int32).reshape(T, k)
    slot[rng.random((T, k)) < rng.uniform(0, 0.3)] = -1
    past = rng.random((T, k)) < 0.02
    slot[past] = rows + rng.integers(0, 1 << 20, int(past.sum()))
    wt = rng.uniform(-1, 1, (T, k)).astype(np.float32)
    y_rows = _bf16(rng.standard_normal((rows, H)))
    keep = (slot.reshape(-1) >= 0) & (slot.reshape(-1) < rows)
    y_pairs = np.zeros((rows, H), np.uint16)
    y_pairs[keep] = y_rows[slot.reshape(-1)[keep]]
    kept = np.where(keep.reshape(T, k), slot, -1).astype(np.int32)
    res_bits = _bf16(rng.standard_normal((T, H)) * rng.choice([1e-20, 1e-3, 1.0, 300.0], (T, 1)))
    gamma_bits = _bf16(rng.uniform(0.25, 2.0, H))
    say(f"[combine+norm random] seed={seed} T={T} H={H} k={k} eps={eps} fp8={fp8}")
    y_dev = to_dev_bf16(y_rows, dev).view(1, rows, H)
    if fp8:
        _check_fp8(f"seed {seed}", dev, y_dev, slot, wt, y_pairs, res_bits, gamma_bits, eps, slot_o=kept)
    else:
        res_g, normed_g = _run(dev, y_dev, slot, wt, res_bits, gamma_bits, eps)
        res_o, normed_o = oracle.combine_residual_rmsnorm(y_pairs, kept, wt, res_bits, gamma_bits, eps)
        _compare(f"seed {seed}", res_g, normed_g, res_o, normed_o)


def test_fp8_output_rejects_bad_sizes(dev):
    y = torch.zeros(1, 8, 192, dtype=torch.bfloat16, device=dev)
    slot = torch.zeros(2, 1, dtype=torch.int32, device=dev)
    w = torch.ones(2, 1, device=dev)
    r = torch.zeros(2, 192, dtype=torch.bfloat16, device=dev)
    g = torch.ones(192, dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoeError):
        moe.moe_combine_residual_rmsnorm_fp8(y, slot, w, r, g)     # H = 192 is not a multiple of 128
