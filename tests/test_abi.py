"""The C ABI without a GPU: the library loads, exports every function include/conv1d.h declares,
and rejects every host-checkable precondition with its status code before launching anything.

The pointers used here are fake, non-overlapping addresses: validation only compares them and never
dereferences them, and every call below fails validation, so no HIP call is reached.
"""
import ctypes
import os
import re

import pytest

from causal_depthwise_conv1d_width_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv1d.h")

OK, EINVAL, EWORKSPACE, EUNSUPPORTED, EHIP, ETOOLARGE = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from causal_depthwise_conv1d_width_amd.build import build
        build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(conv1d_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("conv1d_fwd", "conv1d_state_update", "conv1d_state_update_spec", "conv1d_bwd"):
        assert required in names
    assert set(names) == set(_lib.SIGNATURES), "binding signatures must cover exactly the header"


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_status_strings(lib):
    for code in (OK, EINVAL, EWORKSPACE, EUNSUPPORTED, EHIP, ETOOLARGE):
        assert lib.conv1d_status_str(code)
    assert b"unknown" in lib.conv1d_status_str(99)


def test_workspace_sizes(lib):
    assert lib.conv1d_fwd_workspace_bytes(32768, 5632, 64) == 0
    assert lib.conv1d_bwd_workspace_bytes(0, 64) == 0
    # one FP32 partial per (row range, tap or bias, channel), rounded up to 256 bytes; the number
    # of ranges is at least one and at most one per row, and bounded by the launch's block budget
    for rows, C in ((1, 1), (16384, 5632), (16384, 4096), (1000, 13), (777, 3), (1 << 20, 1), (5, 100000)):
        need = lib.conv1d_bwd_workspace_bytes(rows, C)
        assert need % 256 == 0
        per_range = 9 * C * 4  # room for any filter width up to 8: 8 tap slots + dbias
        ranges = [n for n in range(1, min(rows, 4096) + 1) if 0 <= need - n * per_range < 256]
        assert ranges and (per_range < 256 or len(ranges) == 1), (rows, C, need)
        n = ranges[0]
        strips = -(-C // 512)
        assert n * strips <= max(4096, strips), (rows, C, n)


# ------------------------------------------------------------------ fake device buffers
BASE = 1 << 40


class Fake:
    """Hands out non-overlapping fake addresses."""

    def __init__(self):
        self.next = BASE

    def __call__(self, nbytes, align=256):
        p = (self.next + align - 1) // align * align
        self.next = p + max(nbytes, 1) + 4096
        return ctypes.c_void_p(p)


def seq_cu(fake, nseq):
    s = _lib.Seq()
    s.cu_seqlens = fake(4 * (nseq + 1))
    s.nseq = nseq
    return s


def pool_hist_layout(fake, slots, C, L):
    p = _lib.Pool()
    p.ptr = fake(slots * C * L * 2)
    p.slots, p.len = slots, L
    p.s_slot, p.s_chan, p.s_pos = C * L, L, 1
    p.cache_indices = fake(4 * 8)
    p.has_initial_state = fake(8)
    return p


def fwd(lib, fake, rows=64, C=64, x_ld=None, y_ld=None, w_dtype=1, act=1, seq="cu", pool=None, hist=None,
        x=True, y=True, w=True, b=None, b_dtype=1, width=4):
    x_ld = C if x_ld is None else x_ld
    y_ld = C if y_ld is None else y_ld
    xp = fake(rows * x_ld * 2) if x is True else x
    yp = fake(rows * y_ld * 2) if y is True else y
    wp = fake(C * 16) if w else None
    if seq == "cu":
        seq = seq_cu(fake, 4)
    return lib.conv1d_fwd(xp, rows, C, x_ld, wp, w_dtype, width, b, b_dtype, None if seq is None else ctypes.byref(seq),
                          None if pool is None else ctypes.byref(pool), None if hist is None else ctypes.byref(hist),
                          act, yp, y_ld, None, 0, None)


def test_fwd_rejects_bad_arguments(lib):
    f = Fake()
    assert fwd(lib, f, C=0) == EINVAL
    assert fwd(lib, f, x_ld=63) == EINVAL
    assert fwd(lib, f, y_ld=10) == EINVAL
    assert fwd(lib, f, w=False) == EINVAL
    assert fwd(lib, f, w_dtype=7) == EINVAL
    assert fwd(lib, f, act=2) == EINVAL
    assert fwd(lib, f, x=None) == EINVAL
    assert fwd(lib, f, y=None) == EINVAL
    assert fwd(lib, f, seq=None) == EINVAL
    assert fwd(lib, f, b=f(256), b_dtype=9) == EINVAL
    assert fwd(lib, f, rows=-1) == EINVAL


def test_width_checks(lib):
    f = Fake()
    assert fwd(lib, f, width=1) == EINVAL
    assert fwd(lib, f, width=9) == EINVAL
    C = 64
    p = pool_hist_layout(f, 8, C, 4)
    assert fwd(lib, f, pool=p, width=3) == EINVAL  # the pool form is width four


def test_fwd_rejects_bad_sequence_forms(lib):
    f = Fake()
    s = seq_cu(f, 3)
    s.seq_idx = f(64 * 4)
    assert fwd(lib, f, seq=s) == EINVAL  # offsets and IDs together
    s = _lib.Seq()
    s.seq_idx, s.seqlen = f(64 * 4), 48
    assert fwd(lib, f, seq=s) == EINVAL  # rows % seqlen != 0
    s = _lib.Seq()
    s.seqlen = 0
    assert fwd(lib, f, seq=s) == EINVAL  # batch-row form needs seqlen >= 1
    s = seq_cu(f, 3)
    s.nseq = -1
    assert fwd(lib, f, seq=s) == EINVAL


def test_fwd_rejects_bad_pools(lib):
    f = Fake()
    C = 64
    assert fwd(lib, f, pool=pool_hist_layout(f, 8, C, 2)) == EINVAL  # len < 3
    p = pool_hist_layout(f, 8, C, 4)
    p.s_chan, p.s_pos = 8, 2
    assert fwd(lib, f, pool=p) == EINVAL  # neither axis contiguous
    p = pool_hist_layout(f, 8, C, 4)
    p.s_slot = C * 4 - 1
    assert fwd(lib, f, pool=p) == EINVAL  # slots overlap
    p = pool_hist_layout(f, 8, C, 4)
    p.s_chan = 3
    assert fwd(lib, f, pool=p) == EINVAL  # history positions of neighbouring channels alias
    p = pool_hist_layout(f, 8, C, 4)
    p.s_chan, p.s_pos = 1, C - 1
    assert fwd(lib, f, pool=p) == EINVAL  # channel-contiguous but positions overlap
    p = pool_hist_layout(f, 8, C, 4)
    p.cache_indices = None
    assert fwd(lib, f, pool=p) == EINVAL
    h = _lib.Hist()
    h.ptr = f(4 * 3 * C * 2)
    assert fwd(lib, f, pool=pool_hist_layout(f, 8, C, 4), hist=h) == EINVAL  # pool and history rows
    s = _lib.Seq()
    s.seq_idx, s.seqlen = f(64 * 4), 64
    assert fwd(lib, f, seq=s, pool=pool_hist_layout(f, 8, C, 4)) == EINVAL  # pool needs host-known nseq
    assert fwd(lib, f, seq=s, hist=h) == EINVAL


def test_fwd_rejects_aliasing(lib):
    f = Fake()
    rows, C = 64, 64
    x = f(rows * C * 2)
    assert fwd(lib, f, x=x, y=ctypes.c_void_p(x.value + 128)) == EINVAL  # out overlaps x
    p = pool_hist_layout(f, 8, C, 4)
    assert fwd(lib, f, pool=p, y=ctypes.c_void_p(p.ptr + 64)) == EINVAL  # out overlaps the pool
    p = pool_hist_layout(f, 8, C, 4)
    assert fwd(lib, f, pool=p, x=ctypes.c_void_p(p.ptr)) == EINVAL  # pool overlaps an input
    s = seq_cu(f, 4)
    assert fwd(lib, f, seq=s, y=ctypes.c_void_p(s.cu_seqlens)) == EINVAL  # out overlaps metadata


def bwd(lib, f, rows=256, C=64, ws_bytes=None, ws=True, dw=True, dhist=None, hist=None, dx=None, dy=None,
        seq="cu", dtail=None):
    if seq == "cu":
        seq = seq_cu(f, 4)
    need = lib.conv1d_bwd_workspace_bytes(rows, C)
    ws_bytes = need if ws_bytes is None else ws_bytes
    return lib.conv1d_bwd(f(rows * C * 2), f(rows * C * 2) if dy is None else dy, rows, C, C, C, f(C * 16), 1, 4,
                          None, 1, ctypes.byref(seq), None if hist is None else ctypes.byref(hist), 1,
                          f(rows * C * 2) if dx is None else dx, C, f(C * 16) if dw else None, None, dhist, dtail,
                          f(need) if ws is True else ws, ws_bytes, None)


def test_bwd_rejects_bad_arguments(lib):
    f = Fake()
    assert bwd(lib, f, ws_bytes=100) == EWORKSPACE
    assert bwd(lib, f, ws=None) == EWORKSPACE
    assert bwd(lib, f, dw=False) == EINVAL
    assert bwd(lib, f, dhist=f(4 * 3 * 64 * 2)) == EINVAL  # d(history) needs history rows
    assert bwd(lib, f, ws=ctypes.c_void_p(f(1 << 20).value + 4)) == EINVAL  # misaligned workspace
    dy = f(256 * 64 * 2)
    assert bwd(lib, f, dy=dy, dx=ctypes.c_void_p(dy.value + 64)) == EINVAL  # dx overlaps dy
    s = _lib.Seq()
    s.seq_idx, s.seqlen = f(256 * 4), 256
    h = _lib.Hist()
    h.ptr = f(4 * 3 * 64 * 2)
    assert bwd(lib, f, seq=s, hist=h) == EINVAL  # history rows need host-known nseq
    dx = f(256 * 64 * 2)
    assert bwd(lib, f, dx=dx, dtail=ctypes.c_void_p(dx.value + 256)) == EINVAL  # d(tail) overlaps dx


def test_noalloc_rejects_bad_arguments_and_oversized_problems(lib):
    """The allocation-free backward validates like conv1d_bwd and refuses, before any HIP call, a
    problem whose partials exceed the library's scratch (20 MiB)."""
    f = Fake()
    def call(rows, C, width=4, dw=True, dhist=None, dx=None):
        seq = seq_cu(f, 4)
        return lib.conv1d_bwd_noalloc(f(rows * C * 2), f(rows * C * 2), rows, C, C, C, f(C * 32), 1, width, None, 1,
                                      ctypes.byref(seq), None, 1, f(rows * C * 2) if dx is None else dx, C,
                                      f(C * 32) if dw else None, None, dhist, None, None)
    assert call(256, 64, dw=False) == EINVAL
    assert call(256, 64, width=9) == EINVAL
    assert call(256, 64, dhist=f(4 * 3 * 64 * 2)) == EINVAL  # d(history) needs history rows
    # one row range of 600000 channels: 9 x 600000 x 4 bytes at width 8 (21.6 MB) > 20 MiB, while
    # widths up to four need 5 x 600000 x 4 = 12 MB (that call would launch: not made here)
    assert call(8, 600000, width=8) == ETOOLARGE
    assert b"scratch" in lib.conv1d_status_str(ETOOLARGE)


def test_combine_rejects_bad_arguments(lib):
    f = Fake()
    C, W, S = 64, 4, 3
    def call(parts=True, bparts=None, S=S, C=C, W=W, dw=True, db=None):
        return lib.conv1d_bwd_combine(f(S * C * W * 4) if parts is True else parts, bparts, S, C, W,
                                      f(C * W * 4) if dw is True else dw, db, None)
    assert call(dw=None) == EINVAL
    assert call(C=0) == EINVAL
    assert call(W=1) == EINVAL and call(W=9) == EINVAL
    assert call(S=-1) == EINVAL
    assert call(parts=None) == EINVAL
    assert call(db=f(C * 4)) == EINVAL  # dbias wanted without its parts
    p = f(S * C * W * 4)
    assert call(parts=p, dw=ctypes.c_void_p(p.value + 64)) == EINVAL  # output overlaps the parts
    assert lib.conv1d_bwd_combine(f(4), None, 1 << 40, 1 << 20, 4, f(4), None, None) == EINVAL


def test_state_update_rejects_bad_arguments(lib):
    f = Fake()
    C = 64
    p = pool_hist_layout(f, 8, C, 4)
    args = lambda pool, y: lib.conv1d_state_update(f(8 * C * 2), 8, C, C, f(C * 16), 1, None, 1,
                                                    None if pool is None else ctypes.byref(pool), 1, y, C, None)
    assert args(None, f(8 * C * 2)) == EINVAL
    p2 = pool_hist_layout(f, 8, C, 2)
    assert args(p2, f(8 * C * 2)) == EINVAL
    assert args(p, ctypes.c_void_p(p.ptr + 32)) == EINVAL


def test_spec_update_rejects_bad_arguments(lib):
    f = Fake()
    C, n, K = 64, 8, 3
    def call(pool, y=None, K=K, acc=None, x=None, nseq=n):
        xp = f(nseq * K * C * 2) if x is None else x
        yp = f(nseq * K * C * 2) if y is None else y
        return lib.conv1d_state_update_spec(xp, nseq, K, C, C, f(C * 16), 1, None, 1,
                                            None if pool is None else ctypes.byref(pool), acc, 1, yp, C, None)
    assert call(None) == EINVAL                                    # pool required
    assert call(pool_hist_layout(f, 16, C, 4)) == EINVAL           # len < K + 2
    assert call(pool_hist_layout(f, 16, C, 5), K=0) == EINVAL      # K >= 1
    p = pool_hist_layout(f, 16, C, 5)
    assert call(p, y=ctypes.c_void_p(p.ptr + 64)) == EINVAL        # out overlaps the pool
    p = pool_hist_layout(f, 16, C, 5)
    y = f(n * K * C * 2)
    assert call(p, y=y, acc=ctypes.c_void_p(y.value + 8)) == EINVAL  # out overlaps num_accepted
    x = f(n * K * C * 2)
    assert call(pool_hist_layout(f, 16, C, 5), x=x, y=ctypes.c_void_p(x.value + 2 * C * K)) == EINVAL
    assert call(pool_hist_layout(f, 16, C, 5), nseq=-1) == EINVAL


def test_channels_first_rejects_bad_arguments(lib):
    f = Fake()
    B, D, T = 2, 16, 64
    def fwd_cf(x=None, y=None, xs=(D * T, T), ys=(D * T, T), w=True, act=1, B=B, D=D, T=T):
        xp = f(B * D * T * 2) if x is None else x
        yp = f(B * D * T * 2) if y is None else y
        return lib.conv1d_fwd_cf(xp, B, D, T, xs[0], xs[1], f(D * 16) if w else None, 1, 4, None, 1, act, yp,
                                 ys[0], ys[1], None)
    assert fwd_cf(w=False) == EINVAL
    assert fwd_cf(act=5) == EINVAL
    assert fwd_cf(D=0) == EINVAL
    assert fwd_cf(xs=(D * T, T - 1)) == EINVAL          # rows of one batch overlap
    assert fwd_cf(ys=(T, T)) == EINVAL                  # batches overlap
    x = f(B * D * T * 2)
    assert fwd_cf(x=x, y=ctypes.c_void_p(x.value + 64)) == EINVAL  # out overlaps x
    need = lib.conv1d_bwd_cf_workspace_bytes(B, D)
    assert need >= B * 5 * D * 4 and need % 256 == 0
    assert lib.conv1d_bwd_cf_workspace_bytes(0, D) == 0
    def bwd_cf(ws_bytes=None, ws=True, dw=True, dx=None, dy=None):
        dyp = f(B * D * T * 2) if dy is None else dy
        dxp = f(B * D * T * 2) if dx is None else dx
        nb = need if ws_bytes is None else ws_bytes
        return lib.conv1d_bwd_cf(f(B * D * T * 2), dyp, B, D, T, D * T, T, D * T, T, f(D * 16), 1, 4, None, 1, 1, dxp,
                                 D * T, T, f(D * 16) if dw else None, None, f(need) if ws is True else ws, nb, None)
    assert bwd_cf(ws_bytes=need - 1) == EWORKSPACE
    assert bwd_cf(ws=None) == EWORKSPACE
    assert bwd_cf(dw=False) == EINVAL
    assert bwd_cf(ws=ctypes.c_void_p(f(need + 64).value + 4)) == EINVAL  # misaligned workspace
    dy = f(B * D * T * 2)
    assert bwd_cf(dy=dy, dx=ctypes.c_void_p(dy.value + 32)) == EINVAL  # dx overlaps dy


def test_sizes_whose_byte_extents_overflow_are_rejected(lib):
    """Sizes and strides whose products would overflow the int64 byte arithmetic fail validation
    (fake pointers: nothing is dereferenced and nothing is launched)."""
    f = Fake()
    big_rows, big_ld = 1 << 40, 1 << 20
    x, y, w = f(4096), f(4096), f(4096)
    seq = seq_cu(f, 4)
    assert lib.conv1d_fwd(x, big_rows, 64, big_ld, w, 1, 4, None, 1, ctypes.byref(seq), None, None, 1, y, 64,
                          None, 0, None) == EINVAL
    assert lib.conv1d_fwd(x, 4, 1 << 60, 1 << 60, w, 1, 4, None, 1, ctypes.byref(seq), None, None, 1, y, 1 << 60,
                          None, 0, None) == EINVAL
    assert lib.conv1d_bwd_workspace_bytes(big_rows, big_ld) == 0
    assert lib.conv1d_bwd(x, f(4096), big_rows, 64, big_ld, 64, w, 1, 4, None, 1, ctypes.byref(seq), None, 1,
                          f(4096), 64, f(4096), None, None, None, f(4096), 4096, None) == EINVAL
    p = pool_hist_layout(f, 8, 64, 4)
    p.s_slot = 1 << 60  # slots far apart: the pool's extent overflows
    assert lib.conv1d_state_update(f(4096), 8, 64, 64, w, 1, None, 1, ctypes.byref(p), 1, f(4096), 64,
                                   None) == EINVAL
    p = pool_hist_layout(f, 8, 64, 6)
    assert lib.conv1d_state_update_spec(f(4096), 1 << 40, 1 << 20, 64, 64, w, 1, None, 1, ctypes.byref(p), None, 1,
                                        f(4096), 64, None) == EINVAL
    T = 64
    assert lib.conv1d_fwd_cf(f(4096), 1 << 31, 1, T, T, T, w, 1, 4, None, 1, 1, f(4096), T, T, None) == EINVAL
    assert lib.conv1d_fwd_cf(f(4096), 2, 1 << 40, T, (1 << 40) * (1 << 20), 1 << 20, w, 1, 4, None, 1, 1, f(4096),
                             T, T, None) == EINVAL
    assert lib.conv1d_bwd_cf_workspace_bytes(1 << 40, 1 << 20) == 0
