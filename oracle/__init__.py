"""CPU oracle for MoE routing, dispatch and combine (ctypes over plain C).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never imports, loads or calls it,
and the two share no code.

Every function here only marshals numpy arrays into ``moe_oracle.c``, where
the definitions live (each cites the page passage it follows).  The arrays
use the same layouts as the HIP path:

* logits float32 [T, E]; idx int32 [T, k]; w float32 [T, k]
* counts int32 [E]; token_slot int32 [T, k] (e*C + r or -1); recv_src int32 [E*C]
* x, y bf16 carried as uint16 bit patterns
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11"]

_lib = None

BF16 = 0
FP8_E4M3 = 1


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into libmoe_oracle.so next to it."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_route_topk.argtypes = [P, i64, i32, i32, P, P]
    lib.oracle_route_topk.restype = ctypes.c_int
    lib.oracle_route_topk_grouped.argtypes = [P, i64, i32, i32, i32, i32, P, P]
    lib.oracle_route_topk_grouped.restype = ctypes.c_int
    lib.oracle_assign_slots.argtypes = [P, i64, i32, i32, i32, P, P, P]
    lib.oracle_assign_slots.restype = ctypes.c_int
    lib.oracle_assign_packed.argtypes = [P, i64, i32, i32, P, P, P]
    lib.oracle_assign_packed.restype = ctypes.c_int
    lib.oracle_quantize_row_fp8.argtypes = [P, i32, P, P]
    lib.oracle_quantize_row_fp8.restype = ctypes.c_int
    lib.oracle_filled_rows.argtypes = [P, i32, i32]
    lib.oracle_filled_rows.restype = i64
    lib.oracle_pack.argtypes = [P, i64, i32, i32, P, P, i32, i32, P, P, P]
    lib.oracle_pack.restype = ctypes.c_int
    lib.oracle_combine_residual_rmsnorm.argtypes = [P, P, P, i64, i32, i32, P, P, ctypes.c_float, P, P]
    lib.oracle_combine_residual_rmsnorm.restype = ctypes.c_int
    lib.oracle_bf16_round_double_n.argtypes = [P, i64, P]
    lib.oracle_bf16_round_double_n.restype = ctypes.c_int
    lib.oracle_combine.argtypes = [P, P, P, i64, i32, i32, P, P]
    lib.oracle_combine.restype = ctypes.c_int
    lib.oracle_bf16_round.argtypes = [ctypes.c_float]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_row_bytes.argtypes = [i32, i32]
    lib.oracle_row_bytes.restype = i64
    lib.oracle_fixed_slot_bytes.argtypes = [i64, i64, i32, i32, i32]
    lib.oracle_fixed_slot_bytes.restype = i64
    lib.oracle_quantize_rows_fp8.argtypes = [P, i64, i32, P, P]
    lib.oracle_quantize_rows_fp8.restype = ctypes.c_int
    lib.oracle_bf16_round_n.argtypes = [P, i64, P]
    lib.oracle_bf16_round_n.restype = None
    lib.oracle_e4m3_encode_n.argtypes = [P, i64, P]
    lib.oracle_e4m3_encode_n.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def route_topk(logits: np.ndarray, k: int):
    """Top-k experts per token (descending logit, ties to lower index) and
    their full-softmax weights.  Returns (idx int32 [T,k], w float32 [T,k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(_load().oracle_route_topk(_ptr(logits), T, E, k, _ptr(idx), _ptr(w)), "route_topk")
    return idx, w


def route_topk_grouped(logits: np.ndarray, k: int, n_groups: int, topk_groups: int):
    """Group-limited top-k: experts form n_groups groups of E/n_groups
    consecutive experts, each scored by the fp32 sum of its two largest
    logits; the k experts are chosen among the topk_groups best groups.
    Weights are the full softmax, as in route_topk.  Returns (idx, w)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(_load().oracle_route_topk_grouped(_ptr(logits), T, E, k, n_groups, topk_groups, _ptr(idx), _ptr(w)),
           "route_topk_grouped")
    return idx, w


def assign_slots(idx: np.ndarray, E: int, capacity: int):
    """Per-expert counts and fixed slots in ascending token order.
    Returns (counts int32 [E], token_slot int32 [T,k], recv_src int32 [E*C])."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    token_slot = np.empty((T, k), np.int32)
    recv_src = np.empty(E * capacity, np.int32)
    _check(_load().oracle_assign_slots(_ptr(idx), T, E, k, capacity, _ptr(counts),
                                       _ptr(token_slot), _ptr(recv_src)), "assign_slots")
    return counts, token_slot, recv_src


def assign_packed(idx: np.ndarray, E: int):
    """Packed, count-sized layout: expert e's rows are offsets[e] ..
    offsets[e+1]-1, in ascending token order.  Returns (offsets int32 [E+1],
    token_slot int32 [T,k] (row of each pair), recv_src int32 [T*k])."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    offsets = np.empty(E + 1, np.int32)
    token_slot = np.empty((T, k), np.int32)
    recv_src = np.empty(T * k, np.int32)
    _check(_load().oracle_assign_packed(_ptr(idx), T, E, k, _ptr(offsets), _ptr(token_slot), _ptr(recv_src)),
           "assign_packed")
    return offsets, token_slot, recv_src


def quantize_row_fp8(x_row_bits: np.ndarray):
    """E4M3 codes (uint8 [H]) and per-128 scales (float32 [H/128]) of one bf16 row."""
    x = _c(x_row_bits, np.uint16).reshape(-1)
    H = x.shape[0]
    codes = np.empty(H, np.uint8)
    scales = np.empty(max(H // 128, 1), np.float32)
    _check(_load().oracle_quantize_row_fp8(_ptr(x), H, _ptr(codes), _ptr(scales)), "quantize_row_fp8")
    return codes, scales


def quantize_rows_fp8(x_bits: np.ndarray):
    """Row-wise quantize_row_fp8 of a bf16 matrix [n, H]: codes uint8 [n, H]
    and scales float32 [n, H/128]."""
    x = _c(x_bits, np.uint16)
    n, H = x.shape
    codes = np.empty((n, H), np.uint8)
    scales = np.empty((n, max(H // 128, 1)), np.float32)
    _check(_load().oracle_quantize_rows_fp8(_ptr(x), n, H, _ptr(codes), _ptr(scales)), "quantize_rows_fp8")
    return codes, scales


def pack(x_bits: np.ndarray, dtype: int, recv_src: np.ndarray, counts: np.ndarray, capacity: int):
    """Contents of every filled slot in ascending slot order.
    Returns (rows, scales or None, slot_of_row int32 [R]); rows are uint16 [R,H]
    (bf16) or uint8 [R,H] (fp8 codes) and scales float32 [R, H/128]."""
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    counts = _c(counts, np.int32)
    recv_src = _c(recv_src, np.int32)
    E = counts.shape[0]
    lib = _load()
    R = int(lib.oracle_filled_rows(_ptr(counts), E, capacity))
    slot_of_row = np.empty(R, np.int32)
    if dtype == BF16:
        rows = np.empty((R, H), np.uint16)
        scales = None
    else:
        rows = np.empty((R, H), np.uint8)
        scales = np.empty((R, H // 128), np.float32)
    _check(lib.oracle_pack(_ptr(x), T, H, dtype, _ptr(recv_src), _ptr(counts), E, capacity,
                           _ptr(rows), _ptr(scales), _ptr(slot_of_row)), "pack")
    return rows, scales, slot_of_row


def combine(y_pairs_bits: np.ndarray, token_slot: np.ndarray, w: np.ndarray, want_acc: bool = False):
    """out[t] = bf16(sum_j w[t,j] * y_pairs[t*k+j]) with fp32 FMA in top-k
    order, skipping j with token_slot < 0.  Returns out uint16 [T,H] (and the
    float32 accumulators if want_acc)."""
    token_slot = _c(token_slot, np.int32)
    T, k = token_slot.shape
    y = _c(y_pairs_bits, np.uint16).reshape(T * k, -1)
    H = y.shape[1]
    w = _c(w, np.float32).reshape(T, k)
    out = np.empty((T, H), np.uint16)
    acc = np.empty((T, H), np.float32) if want_acc else None
    _check(_load().oracle_combine(_ptr(y), _ptr(token_slot), _ptr(w), T, k, H, _ptr(out), _ptr(acc)),
           "combine")
    return (out, acc) if want_acc else out


def combine_residual_rmsnorm(y_pairs_bits: np.ndarray, token_slot: np.ndarray, w: np.ndarray,
                             residual_bits: np.ndarray, gamma_bits: np.ndarray, eps: float):
    """Combine, then r = sum + residual (fp32), residual_out = bf16(r) and
    normed_out = bf16(r / sqrt(mean(r^2) + eps) * gamma) (double, one
    rounding).  Returns (residual_out uint16 [T,H], normed_out uint16 [T,H])."""
    token_slot = _c(token_slot, np.int32)
    T, k = token_slot.shape
    y = _c(y_pairs_bits, np.uint16).reshape(T * k, -1)
    H = y.shape[1]
    w = _c(w, np.float32).reshape(T, k)
    res = _c(residual_bits, np.uint16).reshape(T, H)
    gamma = _c(gamma_bits, np.uint16).reshape(H)
    res_out = np.empty((T, H), np.uint16)
    normed = np.empty((T, H), np.uint16)
    _check(_load().oracle_combine_residual_rmsnorm(_ptr(y), _ptr(token_slot), _ptr(w), T, k, H, _ptr(res),
                                                   _ptr(gamma), float(eps), _ptr(res_out), _ptr(normed)),
           "combine_residual_rmsnorm")
    return res_out, normed


def bf16_round_double_array(a: np.ndarray) -> np.ndarray:
    """bf16 RNE bit patterns of float64 values, rounded in one step."""
    flat = _c(a, np.float64).reshape(-1)
    out = np.empty(flat.size, np.uint16)
    _check(_load().oracle_bf16_round_double_n(_ptr(flat), flat.size, _ptr(out)), "bf16_round_double")
    return out.reshape(np.shape(a))


def bf16_round(f: float) -> int:
    return int(_load().oracle_bf16_round(float(f)))


def bf16_round_array(a: np.ndarray) -> np.ndarray:
    flat = _c(a, np.float32).reshape(-1)
    out = np.empty(flat.size, np.uint16)
    _load().oracle_bf16_round_n(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(a))


def e4m3_encode(f: float) -> int:
    return int(_load().oracle_e4m3_encode(float(f)))


def e4m3_encode_array(a: np.ndarray) -> np.ndarray:
    flat = _c(a, np.float32).reshape(-1)
    out = np.empty(flat.size, np.uint8)
    _load().oracle_e4m3_encode_n(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(a))


def row_bytes(H: int, dtype: int) -> int:
    return int(_load().oracle_row_bytes(H, dtype))


def fixed_slot_bytes(experts: int, slots_per_expert: int, H: int, dtype: int, header_bytes: int = 0) -> int:
    return int(_load().oracle_fixed_slot_bytes(experts, slots_per_expert, H, dtype, header_bytes))


# ---------------------------------------------------------------------------
# Range forms for the benchmark's host-cores baseline: the same C functions,
# called on disjoint token (or expert) ranges of preallocated arrays so that
# several threads can run them at once (ctypes releases the GIL for the
# duration of each call).  Marshalling only: no arithmetic here.
# ---------------------------------------------------------------------------

def route_topk_range(logits: np.ndarray, k: int, idx: np.ndarray, w: np.ndarray, t0: int, t1: int):
    """route_topk of tokens t0 .. t1-1, written into rows t0 .. t1-1 of idx and w."""
    T, E = logits.shape
    assert logits.dtype == np.float32 and logits.flags.c_contiguous and 0 <= t0 <= t1 <= T
    assert idx.shape == (T, k) and w.shape == (T, k) and idx.flags.c_contiguous and w.flags.c_contiguous
    _check(_load().oracle_route_topk(_ptr(logits) + t0 * E * 4, t1 - t0, E, k, _ptr(idx) + t0 * k * 4,
                                     _ptr(w) + t0 * k * 4), "route_topk")


def pack_range(x_bits: np.ndarray, dtype: int, recv_src: np.ndarray, counts: np.ndarray, capacity: int,
               rows: np.ndarray, scales: np.ndarray | None, slot_of_row: np.ndarray, e0: int, e1: int, p0: int):
    """pack() of experts e0 .. e1-1 only, written from row p0 of the dense
    outputs (p0 = the filled rows of experts below e0).  slot_of_row holds
    slots relative to expert e0 (add e0 * capacity for the absolute slot)."""
    T, H = x_bits.shape
    E = counts.shape[0]
    assert 0 <= e0 <= e1 <= E and x_bits.flags.c_contiguous
    if e1 == e0:
        return
    row_bytes = H * (2 if dtype == BF16 else 1)
    _check(_load().oracle_pack(_ptr(x_bits), T, H, dtype, _ptr(recv_src) + e0 * capacity * 4, _ptr(counts) + e0 * 4,
                               e1 - e0, capacity, _ptr(rows) + p0 * row_bytes,
                               None if scales is None else _ptr(scales) + p0 * (H // 128) * 4,
                               _ptr(slot_of_row) + p0 * 4), "pack")


def combine_range(y_pairs_bits: np.ndarray, token_slot: np.ndarray, w: np.ndarray, out: np.ndarray, t0: int,
                  t1: int):
    """combine() of tokens t0 .. t1-1, written into rows t0 .. t1-1 of out."""
    T, k = token_slot.shape
    H = out.shape[1]
    assert 0 <= t0 <= t1 <= T and y_pairs_bits.shape == (T * k, H) and out.shape == (T, H)
    for a in (y_pairs_bits, token_slot, w, out):
        assert a.flags.c_contiguous
    if t1 == t0:
        return
    _check(_load().oracle_combine(_ptr(y_pairs_bits) + t0 * k * H * 2, _ptr(token_slot) + t0 * k * 4,
                                  _ptr(w) + t0 * k * 4, t1 - t0, k, H, _ptr(out) + t0 * H * 2, None), "combine")


def combine_residual_rmsnorm_range(y_pairs_bits: np.ndarray, token_slot: np.ndarray, w: np.ndarray,
                                   residual_bits: np.ndarray, gamma_bits: np.ndarray, eps: float,
                                   residual_out: np.ndarray, normed_out: np.ndarray, t0: int, t1: int):
    """combine_residual_rmsnorm() of tokens t0 .. t1-1, written into those
    rows of residual_out and normed_out."""
    T, k = token_slot.shape
    H = normed_out.shape[1]
    assert 0 <= t0 <= t1 <= T and y_pairs_bits.shape == (T * k, H) and residual_bits.shape == (T, H)
    for a in (y_pairs_bits, token_slot, w, residual_bits, gamma_bits, residual_out, normed_out):
        assert a.flags.c_contiguous
    if t1 == t0:
        return
    _check(_load().oracle_combine_residual_rmsnorm(
        _ptr(y_pairs_bits) + t0 * k * H * 2, _ptr(token_slot) + t0 * k * 4, _ptr(w) + t0 * k * 4, t1 - t0, k, H,
        _ptr(residual_bits) + t0 * H * 2, _ptr(gamma_bits), float(eps), _ptr(residual_out) + t0 * H * 2,
        _ptr(normed_out) + t0 * H * 2), "combine_residual_rmsnorm")


def quantize_rows_fp8_range(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, r0: int, r1: int):
    """quantize_rows_fp8() of rows r0 .. r1-1, written into those rows of
    codes and scales."""
    n, H = x_bits.shape
    assert 0 <= r0 <= r1 <= n and codes.shape == (n, H) and scales.shape == (n, H // 128)
    for a in (x_bits, codes, scales):
        assert a.flags.c_contiguous
    if r1 == r0:
        return
    _check(_load().oracle_quantize_rows_fp8(_ptr(x_bits) + r0 * H * 2, r1 - r0, H, _ptr(codes) + r0 * H,
                                            _ptr(scales) + r0 * (H // 128) * 4), "quantize_rows_fp8")


def run_pipeline(logits: np.ndarray, x_bits: np.ndarray, k: int, capacity: int, dtype: int,
                 y_pairs_bits: np.ndarray | None = None):
    """Route, assign slots, pack and (if y_pairs given) combine, all on the CPU."""
    E = logits.shape[1]
    idx, w = route_topk(logits, k)
    counts, token_slot, recv_src = assign_slots(idx, E, capacity)
    rows, scales, slot_of_row = pack(x_bits, dtype, recv_src, counts, capacity)
    res = dict(idx=idx, w=w, counts=counts, token_slot=token_slot, recv_src=recv_src,
               rows=rows, scales=scales, slot_of_row=slot_of_row)
    if y_pairs_bits is not None:
        res["out"] = combine(y_pairs_bits, token_slot, w)
    return res
