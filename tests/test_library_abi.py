"""The HIP library loads on any host, exports every entry point its header
declares, rejects bad arguments on the host before touching a device, and
links nothing from the oracle.  No kernel runs here (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import combine_moe_route_amd as moe
from combine_moe_route_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")]


def _declared():
    names = []
    for h in HEADERS:
        text = open(h).read()
        names += re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        moe.build()
    return moe.load()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("moe_route_topk", "moe_route_topk_grouped", "moe_dispatch", "moe_dispatch_packed", "moe_route_dispatch", "moe_route_dispatch_packed",
              "moe_combine",
              "moe_combine_residual_rmsnorm", "moe_combine_residual_rmsnorm_fp8", "moe_dispatch_workspace_bytes",
              "moe_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", out, re.M))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)
    # nothing but the declared C ABI is exported under the moe_ prefix
    assert {s for s in exported if s.startswith("moe_")} == set(_declared())


def test_library_does_not_link_the_oracle():
    out = subprocess.run(["ldd", LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out
    syms = subprocess.run(["nm", "-D", LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle_" not in syms


def test_status_strings(lib):
    assert moe.moe_status_string(0) == "ok"
    assert "workspace" in moe.moe_status_string(-3)
    assert moe.moe_status_string(99) == "unknown status"


def test_workspace_size(lib):
    assert moe.moe_dispatch_workspace_bytes(32768, 128, 8) == 128 * 128 * 4 + 32768 * 8 * 4
    assert moe.moe_dispatch_workspace_bytes(-1, 8, 2) == 0
    assert moe.moe_dispatch_workspace_bytes(10, 2000, 2) == 0
    assert moe.moe_dispatch_workspace_bytes(0, 8, 2) == 0


def test_host_validation_without_device(lib):
    # every call below fails its argument checks before any HIP call
    P = None
    assert lib.moe_route_topk(P, -1, 8, 2, P, P, P) == -1
    assert lib.moe_route_topk(P, 4, 8, 0, P, P, P) == -1
    assert lib.moe_route_topk(P, 4, 8, 9, P, P, P) == -1
    assert lib.moe_route_topk(P, 4, 4096, 2, P, P, P) == -2
    assert lib.moe_route_topk(P, 4, 64, 17, P, P, P) == -2
    assert lib.moe_route_topk(P, 4, 8, 2, P, P, P) == -1          # null pointers
    assert lib.moe_route_topk(P, 0, 8, 2, P, P, P) == 0           # empty: nothing to do
    g = lib.moe_route_topk_grouped
    assert g(P, 4, 256, 8, 8, 4, P, P, P) == -1                     # null pointers
    assert g(P, 0, 256, 8, 8, 4, P, P, P) == 0                      # empty
    assert g(P, 4, 256, 8, 3, 2, P, P, P) == -1                     # E % n_groups
    assert g(P, 4, 256, 8, 256, 4, P, P, P) == -1                   # groups of one expert
    assert g(P, 4, 256, 8, 8, 0, P, P, P) == -1                     # no group kept
    assert g(P, 4, 256, 8, 8, 9, P, P, P) == -1                     # more kept than groups
    assert g(P, 4, 256, 8, 64, 1, P, P, P) == -1                    # k above the kept experts (1 x 4)
    assert g(P, 4, 1024, 8, 128, 8, P, P, P) == -2                  # more than MOE_MAX_GROUPS groups
    assert g(P, 4, 256, 0, 8, 4, P, P, P) == -1                     # k = 0
    assert lib.moe_combine(P, 8, 4, 64, P, P, -1, 2, P, P) == -1
    assert lib.moe_combine(P, 8, 4, 60, P, P, 4, 2, P, P) == -2
    assert lib.moe_combine(P, 8, 4, 64, P, P, 4, 17, P, P) == -2
    assert lib.moe_combine(P, 8, 4, 64, P, P, 0, 2, P, P) == 0
    assert lib.moe_combine(P, 8, 4, 64, P, P, 4, 2, P, P) == -1
    assert lib.moe_combine(P, 65536, 65536, 64, P, P, 4, 2, P, P) == -2   # E*C beyond int32
    cn = lib.moe_combine_residual_rmsnorm
    A = 1 << 20                                                      # fake, 16 B aligned addresses (never used)
    assert cn(P, 8, 4, 64, P, P, 4, 2, P, P, 1e-6, P, P, P) == -1     # null pointers
    assert cn(P, 8, 4, 64, P, P, 0, 2, P, P, 1e-6, P, P, P) == 0      # empty
    assert cn(P, 8, 4, 64, P, P, 4, 2, P, P, -1.0, P, P, P) == -1     # eps < 0
    assert cn(P, 8, 4, 64, P, P, 4, 2, P, P, float("nan"), P, P, P) == -1
    assert cn(P, 8, 4, 60, P, P, 4, 2, P, P, 1e-6, P, P, P) == -2     # H % 8
    assert cn(P, 8, 4, 16392, P, P, 4, 2, P, P, 1e-6, P, P, P) == -2  # H above MOE_MAX_NORM_HIDDEN
    assert cn(P, 8, 4, 64, P, P, 4, 17, P, P, 1e-6, P, P, P) == -2    # k above MOE_MAX_TOPK
    # normed_out overlapping y, residual_out overlapping residual (not equal): rejected before any launch
    assert cn(A, 8, 4, 64, A + 4096, A + 8192, 4, 2, A + 2 * 4096, A + 3 * 4096, 1e-6, A + 4 * 4096, A + 256,
              P) == -1
    assert cn(A, 8, 4, 64, A + 8192, A + 12288, 4, 2, A + 4 * 4096, A + 5 * 4096, 1e-6, A + 4 * 4096 + 16,
              A + 7 * 4096, P) == -1
    cq = lib.moe_combine_residual_rmsnorm_fp8
    assert cq(P, 8, 4, 192, P, P, 4, 2, P, P, 1e-6, P, P, P, P, P) == -2   # H % 128
    assert cq(P, 8, 4, 256, P, P, 0, 2, P, P, 1e-6, P, P, P, P, P) == 0    # empty
    assert cq(P, 8, 4, 256, P, P, 4, 2, P, P, 1e-6, P, P, P, P, P) == -1   # null pointers
    K = 1024                                                           # y [8][4][256] bf16 = 16 KiB at A
    args = dict(ts=A + 16 * K, tw=A + 16 * K + 256, res=A + 20 * K, g=A + 24 * K, ro=A + 28 * K)
    def cq_at(q, sc, normed=None):
        return cq(A, 8, 4, 256, args["ts"], args["tw"], 4, 2, args["res"], args["g"], 1e-6, args["ro"], normed, q,
                  sc, P)
    assert cq_at(A + 32 * K, A + 32 * K + 512) == -1                  # scales inside the codes [4][256]
    assert cq_at(A + 32 * K + 4, A + 34 * K) == -1                    # codes not 8 B aligned
    assert cq_at(A + 32 * K, A + 34 * K + 2) == -1                    # scales not 4 B aligned
    assert cq_at(A + 32 * K, A + 34 * K, normed=A + 33 * K) == -1     # bf16 rows overlapping the scales
    assert cq_at(A + 8 * K, A + 34 * K) == -1                         # codes overlapping y
    assert cq_at(A + 32 * K, args["ts"]) == -1                        # scales overlapping token_slot
    rd = lib.moe_route_dispatch
    assert rd(P, 4, 8, 2, P, 64, 4, 0, P, P, P, P, P, P, P, P, 0, P) == -1    # null pointers
    assert rd(P, 4, 8, 9, P, 64, 4, 0, P, P, P, P, P, P, P, P, 0, P) == -1    # k > E
    assert rd(P, 4, 8, 2, P, 64, 0, 0, P, P, P, P, P, P, P, P, 0, P) == -1    # capacity 0
    assert rd(P, 4, 8, 2, P, 100, 4, 0, P, P, P, P, P, P, P, P, 0, P) == -2   # H % 8
    assert rd(P, 4, 8, 2, P, 192, 4, 1, P, P, P, P, P, P, P, P, 0, P) == -2   # fp8 needs H % 128
    assert rd(P, 4, 4096, 2, P, 64, 4, 0, P, P, P, P, P, P, P, P, 0, P) == -2 # E above the limit
    rp = lib.moe_route_dispatch_packed
    assert rp(P, 4, 8, 2, P, 64, 0, P, P, P, P, P, P, P, P, 0, P) == -1        # null pointers
    assert rp(P, 4, 8, 9, P, 64, 0, P, P, P, P, P, P, P, P, 0, P) == -1        # k > E
    assert rp(P, 4, 8, 2, P, 100, 0, P, P, P, P, P, P, P, P, 0, P) == -2       # H % 8
    assert rp(P, 4, 8, 2, P, 192, 1, P, P, P, P, P, P, P, P, 0, P) == -2       # fp8 needs H % 128
    assert rp(P, 4, 8, 2, P, 64, 2, P, P, P, P, P, P, P, P, 0, P) == -1        # bad dtype
    assert rp(P, 1 << 25, 8, 2, P, 64, 0, P, P, P, P, P, P, P, P, 0, P) == -2  # T above the limit
    pk = lib.moe_dispatch_packed
    assert pk(P, 4, 64, P, 8, 2, 0, P, P, P, P, P, P, 0, P) == -1        # null pointers
    assert pk(P, 4, 64, P, 8, 2, 2, P, P, P, P, P, P, 0, P) == -1        # bad dtype
    assert pk(P, 4, 100, P, 8, 2, 0, P, P, P, P, P, P, 0, P) == -2       # H % 8
    assert pk(P, 4, 192, P, 8, 2, 1, P, P, P, P, P, P, 0, P) == -2       # fp8 needs H % 128
    assert pk(P, 4, 64, P, 8, 9, 0, P, P, P, P, P, P, 0, P) == -1        # k > E
    assert pk(P, 1 << 25, 64, P, 8, 2, 0, P, P, P, P, P, P, 0, P) == -2  # T above the limit
    d = lib.moe_dispatch
    assert d(P, 4, 64, P, 8, 2, 4, 0, P, P, P, P, P, P, 0, P) == -1     # null pointers
    assert d(P, 4, 64, P, 8, 2, 4, 2, P, P, P, P, P, P, 0, P) == -1     # bad dtype
    assert d(P, 4, 64, P, 8, 2, 0, 0, P, P, P, P, P, P, 0, P) == -1     # capacity 0
    assert d(P, 4, 100, P, 8, 2, 4, 0, P, P, P, P, P, P, 0, P) == -2    # H % 8
    assert d(P, 4, 192, P, 8, 2, 4, 1, P, P, P, P, P, P, 0, P) == -2    # fp8 needs H % 128
    assert d(P, 4, 64, P, 8, 9, 4, 0, P, P, P, P, P, P, 0, P) == -1     # k > E


def _fake_layout(*sizes):
    """Fake, 256 B aligned, non-overlapping device addresses for buffers of
    the given byte sizes (never dereferenced)."""
    addr, out = 1 << 20, []
    for n in sizes:
        out.append(addr)
        addr += (n + 255) // 256 * 256 + 256
    return out


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="passes fake device addresses; host-only check")
def test_grids_beyond_one_launch_are_unsupported(lib):
    """A dispatch or combine whose single launch would need more than 2^32 - 1
    work-items is refused on the host with MOE_ERR_UNSUPPORTED before
    anything is enqueued (T = 2^24 tokens of 65536 elements)."""
    T, E, k = 1 << 24, 8, 2
    ws = moe.moe_dispatch_workspace_bytes(T, E, k)
    assert ws > 0
    d = lib.moe_dispatch

    def dispatch(H, dtype, packed=False):
        rows = T * k if packed else E * T
        row = H if dtype else 2 * H
        x, idx, rx, sc, src, cnt, slot, w = _fake_layout(T * H * 2, T * k * 4, rows * row, rows * (H // 128) * 4,
                                                         rows * 4, (E + 1) * 4, T * k * 4, ws)
        if packed:
            return lib.moe_dispatch_packed(x, T, H, idx, E, k, dtype, rx, sc if dtype else None, src, cnt, slot, w,
                                           ws, None)
        return d(x, T, H, idx, E, k, T, dtype, rx, sc if dtype else None, src, cnt, slot, w, ws, None)

    H = 65536
    assert dispatch(H, 0) == -2
    assert dispatch(H, 1) == -2
    assert dispatch(H, 0, packed=True) == -2
    lg, x, idx, tw, rx, src, cnt, slot, w = _fake_layout(T * E * 4, T * H * 2, T * k * 4, T * k * 4, E * T * 2 * H,
                                                         E * T * 4, E * 4, T * k * 4, ws)
    assert lib.moe_route_dispatch(lg, T, E, k, x, H, T, 0, idx, tw, rx, None, src, cnt, slot, w, ws, None) == -2
    # combine: y of E x C rows, out placed after it
    y, ts, tw, out = _fake_layout(E * 4 * H * 2, T * k * 4, T * k * 4, T * H * 2)
    assert lib.moe_combine(y, E, 4, H, ts, tw, T, k, out, None) == -2
    # control: at H = 4096 the same calls pass every host check and reach the
    # launch, which fails with MOE_ERR_HIP on a host without a GPU
    assert dispatch(4096, 0) == -4
    y, ts, tw, out = _fake_layout(E * 4 * 4096 * 2, T * k * 4, T * k * 4, T * 4096 * 2)
    assert lib.moe_combine(y, E, 4, 4096, ts, tw, T, k, out, None) == -4


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="passes fake device addresses; host-only check")
def test_overlapping_buffers_are_rejected(lib):
    """Every entry point refuses an output that overlaps an input or another
    output, on the host, before anything is enqueued."""
    T, E, k, H = 64, 8, 2, 256
    ws = moe.moe_dispatch_workspace_bytes(T, E, k)
    lg, x, idx, tw, rx, sc, src, cnt, slot, w = _fake_layout(T * E * 4, T * H * 2, T * k * 4, T * k * 4,
                                                             E * T * H * 2, E * T * (H // 128) * 4, E * T * 4,
                                                             (E + 1) * 4, T * k * 4, ws)
    r = lib.moe_route_topk
    assert r(lg, T, E, k, lg + 64, tw, None) == -1                       # ids inside the logits
    assert r(lg, T, E, k, idx, idx + 64, None) == -1                     # weights inside the ids
    assert lib.moe_route_topk_grouped(lg, T, E, k, 2, 1, idx, lg, None) == -1
    d = lib.moe_dispatch
    assert d(x, T, H, idx, E, k, T, 0, rx, None, src, cnt, slot, w, ws, None) == -4    # control (no GPU)
    assert d(x, T, H, idx, E, k, T, 0, x + 512, None, src, cnt, slot, w, ws, None) == -1  # rows over x
    assert d(x, T, H, idx, E, k, T, 0, rx, None, src, cnt, idx, w, ws, None) == -1        # slots over ids
    assert d(x, T, H, idx, E, k, T, 0, rx, None, src, cnt, slot, src, ws, None) == -1     # workspace over src
    assert d(x, T, H, idx, E, k, T, 1, rx, rx + 4096, src, cnt, slot, w, ws, None) == -1  # scales inside codes
    pk = lib.moe_dispatch_packed
    assert pk(x, T, H, idx, E, k, 0, rx, None, src, src + 8, slot, w, ws, None) == -1     # offsets inside src
    rd = lib.moe_route_dispatch
    assert rd(lg, T, E, k, x, H, T, 0, idx, tw, rx, None, src, cnt, slot, w, ws, None) == -4  # control
    assert rd(lg, T, E, k, x, H, T, 0, idx, lg, rx, None, src, cnt, slot, w, ws, None) == -1  # weights over logits
    assert rd(lg, T, E, k, x, H, T, 0, idx, tw, rx, None, src, cnt, tw, w, ws, None) == -1   # slots over weights
    rp = lib.moe_route_dispatch_packed
    assert rp(lg, T, E, k, x, H, 0, idx, tw, rx, None, src, rx + 1024, slot, w, ws, None) == -1
    c = lib.moe_combine
    y, out = rx, x
    assert c(y, E, T, H, slot, tw, T, k, out, None) == -4                # control
    assert c(y, E, T, H, slot, tw, T, k, slot, None) == -1               # out over the slots


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="passes fake device addresses; host-only check")
def test_noalloc_checks_before_any_hip_call(lib):
    """moe_route_dispatch_noalloc checks its arguments, then the batch's
    workspace need against its static scratch (MOE_ERR_SCRATCH), all on the
    host before the scratch address is looked up or anything is enqueued."""
    na = lib.moe_route_dispatch_noalloc
    P = None
    assert na(P, 4, 8, 2, P, 64, 4, 0, P, P, P, P, P, P, P, P) == -1       # null pointers
    assert na(P, 4, 8, 9, P, 64, 4, 0, P, P, P, P, P, P, P, P) == -1       # k > E
    assert na(P, 4, 8, 2, P, 64, 0, 0, P, P, P, P, P, P, P, P) == -1       # capacity 0
    assert na(P, 4, 8, 2, P, 100, 4, 0, P, P, P, P, P, P, P, P) == -2      # H % 8
    assert na(P, 4, 4096, 2, P, 64, 4, 0, P, P, P, P, P, P, P, P) == -2    # E above the limit

    def call(T, E, k, H=128):
        lg, x, idx, tw, rx, src, cnt, slot = _fake_layout(T * E * 4, T * H * 2, T * k * 4, T * k * 4,
                                                          E * T * 2 * H, E * T * 4, E * 4, T * k * 4)
        return na(lg, T, E, k, x, H, T, 0, idx, tw, rx, None, src, cnt, slot, None)

    limit = moe.MOE_NOALLOC_SCRATCH_BYTES
    assert moe.moe_dispatch_workspace_bytes(200_000, 16, 8) > limit
    assert call(200_000, 16, 8) == moe.binding.MOE_ERR_SCRATCH
    assert "scratch" in moe.moe_status_string(moe.binding.MOE_ERR_SCRATCH)
    # a batch within the limit passes every host check and fails only at the
    # scratch lookup (no GPU here): MOE_ERR_HIP
    assert moe.moe_dispatch_workspace_bytes(4096, 16, 8) <= limit
    assert call(4096, 16, 8) == -4
