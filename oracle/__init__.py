"""ctypes wrapper of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()`` and by the
benchmark's CPU-baseline leg, never by the library.  bf16 tensors are numpy ``uint16`` arrays of
bit patterns; taps and bias are ``float32`` (FP32) or ``uint16`` (bf16 bits) arrays.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


class OracleError(ValueError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data


def _row_major_2d(a, name):
    if a.ndim == 2 and a.size == 0:
        return max(a.shape[1], 1)
    if a.ndim == 2 and a.shape[1] == 1 and a.strides[0] > 0 and a.strides[0] % a.itemsize == 0:
        return a.strides[0] // a.itemsize
    if a.ndim != 2 or a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
        raise OracleError(f"{name}: need a 2-D array with contiguous channels")
    return a.strides[0] // a.itemsize


def _taps(w, C, name, shape):
    if w is None:
        return None, 0
    if w.shape != shape or not w.flags.c_contiguous:
        raise OracleError(f"{name}: need a contiguous array of shape {shape}")
    if w.dtype == np.float32:
        return w, 1
    if w.dtype == np.uint16:
        return w, 0
    raise OracleError(f"{name}: dtype must be float32 or uint16 (bf16 bits)")


def _width(w, C):
    """Taps [C, W] with W in 2..8 (the width of the depthwise filter)."""
    if w is None or w.ndim != 2 or w.shape[0] != C or not 2 <= w.shape[1] <= 8:
        raise OracleError("weight: need taps of shape [C, W] with 2 <= W <= 8")
    return int(w.shape[1])


class Oracle:
    def __init__(self, path=DEFAULT_LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} missing: run `python oracle/build.py`")
        lib = ctypes.CDLL(path)
        lib.oracle_fwd.argtypes = [_p, _i64, _i64, _i64, _p, _int, _int, _p, _int, _p, _i64, _p, _i64,
                                   _p, _i64, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _int, _p,
                                   _i64, _int]
        lib.oracle_fwd.restype = _int
        lib.oracle_bwd.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _p, _int, _int, _p, _int, _p, _i64,
                                   _p, _i64, _p, _p, _int, _p, _i64, _p, _p, _p, _p, _int]
        lib.oracle_bwd.restype = _int
        lib.oracle_state_update.argtypes = [_p, _i64, _i64, _i64, _p, _int, _p, _int, _p, _i64,
                                            _i64, _i64, _i64, _i64, _p, _int, _p, _i64]
        lib.oracle_state_update.restype = _int
        lib.oracle_spec_update.argtypes = [_p, _i64, _i64, _i64, _i64, _p, _int, _p, _int, _p, _i64,
                                           _i64, _i64, _i64, _i64, _p, _p, _int, _p, _i64]
        lib.oracle_spec_update.restype = _int
        lib.oracle_combine.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_combine.restype = _int
        lib.oracle_round_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_round_float_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_round_float_to_bf16.restype = ctypes.c_uint16
        lib.oracle_max_threads.restype = _int
        self.lib = lib
        self.path = path

    # ------------------------------------------------------------------ helpers
    @staticmethod
    def _seq(rows, cu_seqlens, seq_idx, seqlen):
        cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        si = None if seq_idx is None else np.ascontiguousarray(seq_idx, dtype=np.int32)
        nseq = 0 if cu is None else cu.shape[0] - 1
        if cu is None and seqlen is None:
            seqlen = max(rows, 1)
        return cu, si, nseq, (0 if seqlen is None else int(seqlen))

    @staticmethod
    def _pool(pool, C):
        if pool is None:
            return None, 0, 0, 0, 0, 0
        if pool.dtype != np.uint16 or pool.ndim != 3 or pool.shape[1] != C:
            raise OracleError("pool: need uint16 [slots, C, L]")
        st = [s // 2 for s in pool.strides]
        return pool, pool.shape[0], pool.shape[2], st[0], st[1], st[2]

    def threads(self):
        return self.lib.oracle_max_threads()

    def round_double(self, d):
        return int(self.lib.oracle_round_double_to_bf16(float(d)))

    def round_float(self, f):
        return int(self.lib.oracle_round_float_to_bf16(float(f)))

    # ------------------------------------------------------------------ forward
    def fwd(self, x, w, b=None, *, cu_seqlens=None, seq_idx=None, seqlen=None, pool=None,
            cache_indices=None, has_initial_state=None, hist=None, has_history=None, act="silu",
            y=None, fill=0x7FC1, nthreads=0):
        """y (uint16 bits) for packed rows x; `pool` is updated in place."""
        x = np.asarray(x)
        rows, C = x.shape
        x_ld = _row_major_2d(x, "x")
        W = _width(np.asarray(w), C)
        w, wf = _taps(w, C, "weight", (C, W))
        b, bf = _taps(b, C, "bias", (C,))
        cu, si, nseq, seqlen = self._seq(rows, cu_seqlens, seq_idx, seqlen)
        pl, slots, L, ss, sc, sp = self._pool(pool, C)
        ci = None if cache_indices is None else np.ascontiguousarray(cache_indices, dtype=np.int32)
        hi = None if has_initial_state is None else np.ascontiguousarray(has_initial_state, dtype=np.uint8)
        hh = None if has_history is None else np.ascontiguousarray(has_history, dtype=np.uint8)
        if hist is not None and (hist.dtype != np.uint16 or not hist.flags.c_contiguous or hist.shape[1:] != (W - 1, C)):
            raise OracleError("hist: need contiguous uint16 [nseq, W - 1, C]")
        if y is None:
            y = np.full((rows, C), fill, dtype=np.uint16)
        y_ld = _row_major_2d(y, "y")
        rc = self.lib.oracle_fwd(_ptr(x), rows, C, x_ld, _ptr(w), wf, W, _ptr(b), bf, _ptr(cu), nseq,
                                 _ptr(si), seqlen, _ptr(pl), slots, L, ss, sc, sp, _ptr(ci),
                                 _ptr(hi), _ptr(hist), _ptr(hh), {"none": 0, "silu": 1}[act],
                                 _ptr(y), y_ld, int(nthreads))
        if rc != 0:
            raise OracleError(f"oracle_fwd rejected its input (code {rc})")
        return y

    # ------------------------------------------------------------------ decode
    def state_update(self, x, w, b=None, *, pool, cache_indices, act="silu", fill=0x7FC1):
        x = np.asarray(x)
        nseq, C = x.shape
        x_ld = _row_major_2d(x, "x")
        w, wf = _taps(w, C, "weight", (C, 4))
        b, bf = _taps(b, C, "bias", (C,))
        pl, slots, L, ss, sc, sp = self._pool(pool, C)
        ci = np.ascontiguousarray(cache_indices, dtype=np.int32)
        y = np.full((nseq, C), fill, dtype=np.uint16)
        rc = self.lib.oracle_state_update(_ptr(x), nseq, C, x_ld, _ptr(w), wf, _ptr(b), bf, _ptr(pl),
                                          slots, L, ss, sc, sp, _ptr(ci), {"none": 0, "silu": 1}[act],
                                          _ptr(y), C)
        if rc != 0:
            raise OracleError(f"oracle_state_update rejected its input (code {rc})")
        return y

    def spec_update(self, x, w, b=None, *, pool, cache_indices, accepted=None, act="silu", fill=0x7FC1):
        """Speculative multi-token update: x [nseq, K, C] bf16 bits, `accepted` [nseq] int32 (None =
        all 1); returns y [nseq, K, C] and updates `pool` in place (see oracle_spec_update)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        if x.ndim != 3:
            raise ValueError("x must be [nseq, K, C]")
        nseq, K, C = x.shape
        w, wf = _taps(w, C, "weight", (C, 4))
        b, bf = _taps(b, C, "bias", (C,))
        pl, slots, L, ss, sc, sp = self._pool(pool, C)
        ci = np.ascontiguousarray(cache_indices, dtype=np.int32)
        acc = None if accepted is None else np.ascontiguousarray(accepted, dtype=np.int32)
        y = np.full((nseq, K, C), fill, dtype=np.uint16)
        rc = self.lib.oracle_spec_update(_ptr(x), nseq, K, C, C, _ptr(w), wf, _ptr(b), bf, _ptr(pl), slots, L,
                                         ss, sc, sp, _ptr(ci), _ptr(acc), {"none": 0, "silu": 1}[act], _ptr(y), C)
        if rc != 0:
            raise OracleError(f"oracle_spec_update rejected its input (code {rc})")
        return y

    # ------------------------------------------------------------------ channels-first layout
    # [B, D, T] with T contiguous: every (b, d) row is one sequence with zero history.  The
    # operation is the channel-last one on the transposed array, so these wrappers transpose to
    # [B*T, D], run the batch-row form (seqlen = T) and transpose back.
    def fwd_cf(self, x, w, b=None, *, act="silu", nthreads=0):
        x = np.asarray(x, dtype=np.uint16)
        B, D, T = x.shape
        if B * T == 0:
            return np.zeros((B, D, T), dtype=np.uint16)
        xl = np.ascontiguousarray(x.transpose(0, 2, 1)).reshape(B * T, D)
        yl = self.fwd(xl, w, b, seqlen=T, act=act, nthreads=nthreads)
        return np.ascontiguousarray(yl.reshape(B, T, D).transpose(0, 2, 1))

    def bwd_cf(self, x, dy, w, b=None, *, act="silu", want_db=None, nthreads=0):
        """(dx bits [B, D, T], dw float32 [D, 4], db float32 [D] or None)."""
        x = np.asarray(x, dtype=np.uint16)
        B, D, T = x.shape
        xl = np.ascontiguousarray(x.transpose(0, 2, 1)).reshape(B * T, D)
        dyl = np.ascontiguousarray(np.asarray(dy, dtype=np.uint16).transpose(0, 2, 1)).reshape(B * T, D)
        dx, dw, db, _ = self.bwd(xl, dyl, w, b, seqlen=max(T, 1), act=act, want_db=want_db, nthreads=nthreads)
        return np.ascontiguousarray(dx.reshape(B, T, D).transpose(0, 2, 1)), dw, db

    # ------------------------------------------------------------------ backward
    def bwd(self, x, dy, w, b=None, *, cu_seqlens=None, seq_idx=None, seqlen=None, hist=None,
            has_history=None, act="silu", want_db=None, want_dhist=None, dtail=None, fill=0x7FC1, nthreads=0):
        """(dx bits, dw float32 [C, W], db float32 [C] or None, dhist bits or None).

        dtail: bf16 bits [W - 1, C] or None, the next shard's gradient of the last W - 1 values of
        the last sequence's extended sequence (see oracle_bwd)."""
        x = np.asarray(x)
        dy = np.asarray(dy)
        rows, C = x.shape
        x_ld = _row_major_2d(x, "x")
        dy_ld = _row_major_2d(dy, "dy")
        W = _width(np.asarray(w), C)
        w, wf = _taps(w, C, "weight", (C, W))
        if hist is not None and (hist.dtype != np.uint16 or not hist.flags.c_contiguous or hist.shape[1:] != (W - 1, C)):
            raise OracleError("hist: need contiguous uint16 [nseq, W - 1, C]")
        b, bf = _taps(b, C, "bias", (C,))
        cu, si, nseq, seqlen = self._seq(rows, cu_seqlens, seq_idx, seqlen)
        hh = None if has_history is None else np.ascontiguousarray(has_history, dtype=np.uint8)
        if want_db is None:
            want_db = b is not None
        if want_dhist is None:
            want_dhist = hist is not None
        dx = np.full((rows, C), fill, dtype=np.uint16)
        dw = np.zeros((C, W), dtype=np.float32)
        db = np.zeros((C,), dtype=np.float32) if want_db else None
        dhist = np.full(hist.shape, fill, dtype=np.uint16) if (want_dhist and hist is not None) else None
        if dtail is not None:
            dtail = np.asarray(dtail)
            if dtail.dtype != np.uint16 or not dtail.flags.c_contiguous or dtail.shape != (W - 1, C):
                raise OracleError("dtail: need contiguous uint16 [W - 1, C]")
        rc = self.lib.oracle_bwd(_ptr(x), _ptr(dy), rows, C, x_ld, dy_ld, _ptr(w), wf, W, _ptr(b), bf,
                                 _ptr(cu), nseq, _ptr(si), seqlen, _ptr(hist), _ptr(hh),
                                 {"none": 0, "silu": 1}[act], _ptr(dx), C, _ptr(dw), _ptr(db),
                                 _ptr(dhist), _ptr(dtail), int(nthreads))
        if rc != 0:
            raise OracleError(f"oracle_bwd rejected its input (code {rc})")
        return dx, dw, db, dhist

    # ------------------------------------------------------------------ shard-ordered combine
    def combine(self, parts):
        """parts: float32 [nshards, ...]; returns the element-wise sum in ascending shard order
        (one FP32 addition per shard, starting from shard 0's value), shaped like one shard."""
        parts = np.ascontiguousarray(parts, dtype=np.float32)
        if parts.ndim < 1:
            raise OracleError("parts: need a leading shard axis")
        nshards = parts.shape[0]
        n = int(np.prod(parts.shape[1:], dtype=np.int64))
        out = np.zeros(parts.shape[1:], dtype=np.float32)
        rc = self.lib.oracle_combine(_ptr(parts), nshards, n, _ptr(out))
        if rc != 0:
            raise OracleError(f"oracle_combine rejected its input (code {rc})")
        return out
