"""Packed width-4 depthwise causal Conv1d (+ SiLU) for MI355X (gfx950).

Thin torch binding of the C ABI in include/conv1d.h: every function below only checks tensor
metadata, marshals pointers, sizes and the current HIP stream, and calls the library; all of
the computation runs in the hand-written HIP kernels of ``csrc/``.  bf16 tensors are
``torch.bfloat16`` (or 16-bit integer views holding bf16 bits); taps and bias are
``torch.float32`` or ``torch.bfloat16``.

Entry points (same names as the C ABI):
  conv1d_fwd           forward over packed rows: cu_seqlens / per-token sequence IDs / batch
                       rows, optional slot pool (conv_state, cache_indices, has_initial_state)
                       or caller history rows (history, has_history)
  conv1d_state_update  one decode step per sequence against its slot
  conv1d_state_update_spec  K speculative tokens per sequence, history read at the accepted offset
  conv1d_bwd           dx, deterministic FP32 dweight / dbias, and d(history); optionally takes the
                       next shard's gradient of this shard's tail (dtail)
  conv1d_bwd_combine   per-shard dweight / dbias contributions added in ascending shard order
  conv1d_bwd_noalloc   conv1d_bwd without a workspace, for callers that cannot allocate: the
                       partials use a scratch array the library holds on each GPU
  conv1d_fwd_cf / conv1d_bwd_cf  the channels-first layout [B, D, T] (T contiguous, one sequence
                       per (b, d) row, zero history)
"""
import ctypes

from . import _lib

__all__ = ["conv1d_fwd", "conv1d_state_update", "conv1d_state_update_spec", "conv1d_bwd", "conv1d_bwd_combine",
           "conv1d_bwd_noalloc", "conv1d_fwd_cf",
           "conv1d_bwd_cf", "conv1d_bwd_cf_workspace_bytes", "conv1d_fwd_workspace_bytes",
           "conv1d_bwd_workspace_bytes", "library_path"]

library_path = _lib.LIB_PATH


def _torch():
    import torch
    return torch


def _bits_ok(t):
    torch = _torch()
    return t.dtype in (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else \
        t.dtype in (torch.bfloat16, torch.int16)


def _rows2d(t, name, C=None):
    if t.dim() != 2 or not _bits_ok(t):
        raise ValueError(f"{name}: need a 2-D bf16 tensor")
    if t.shape[0] > 0 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: channels must be contiguous")
    if C is not None and t.shape[1] != C:
        raise ValueError(f"{name}: expected {C} channels")
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    return t.data_ptr(), max(ld, t.shape[1])


def _taps(t, C, shape, name):
    torch = _torch()
    if t is None:
        return None, 0
    if tuple(t.shape) != shape or not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous tensor of shape {shape}")
    if t.dtype == torch.float32:
        return t.data_ptr(), _lib.F32
    if t.dtype == torch.bfloat16:
        return t.data_ptr(), _lib.BF16
    raise ValueError(f"{name}: dtype must be float32 or bfloat16")


def _i32(t, name):
    torch = _torch()
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous int32 tensor")
    return t.data_ptr()


def _u8(t, name):
    torch = _torch()
    if t is None:
        return None
    if t.dtype not in (torch.bool, torch.uint8) or not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous bool/uint8 tensor")
    return t.data_ptr()


def _seq(rows, cu_seqlens, seq_idx, seqlen):
    s = _lib.Seq()
    if cu_seqlens is not None:
        s.cu_seqlens = _i32(cu_seqlens, "cu_seqlens")
        s.nseq = cu_seqlens.numel() - 1
        return s, s.nseq
    s.seq_idx = _i32(seq_idx, "seq_idx")
    s.seqlen = int(seqlen) if seqlen is not None else max(rows, 1)
    return s, (rows // s.seqlen if seq_idx is None else -1)


def _pool(conv_state, cache_indices, has_initial_state, C):
    if conv_state is None:
        return None
    if conv_state.dim() != 3 or conv_state.shape[1] != C or not _bits_ok(conv_state):
        raise ValueError("conv_state: need a bf16 [slots, C, L] tensor")
    p = _lib.Pool()
    p.ptr = conv_state.data_ptr()
    p.slots, _, p.len = conv_state.shape
    p.s_slot, p.s_chan, p.s_pos = conv_state.stride()
    if conv_state.shape[0] == 1:
        p.s_slot = max(p.s_slot, 1)
    p.cache_indices = _i32(cache_indices, "cache_indices")
    p.has_initial_state = _u8(has_initial_state, "has_initial_state")
    return p


def _width(weight, C, max_width=8):
    """Filter width W from taps [C, W], W in 2..max_width."""
    if weight is None or weight.dim() != 2 or weight.shape[0] != C or not 2 <= weight.shape[1] <= max_width:
        raise ValueError(f"weight: need taps of shape [{C}, W] with 2 <= W <= {max_width}")
    return int(weight.shape[1])


def _hist(history, has_history, C, W=4):
    if history is None:
        return None
    if history.dim() != 3 or tuple(history.shape[1:]) != (W - 1, C) or not history.is_contiguous() or not _bits_ok(history):
        raise ValueError(f"history: need a contiguous bf16 [nseq, {W - 1}, C] tensor")
    h = _lib.Hist()
    h.ptr = history.data_ptr()
    h.has_history = _u8(has_history, "has_history")
    return h


def _stream(stream, dev):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return ctypes.c_void_p(stream.cuda_stream)


def _on_gpu(dev, **tensors):
    """Every tensor argument must live on x's GPU: the kernels dereference the raw pointers."""
    if dev.type != "cuda":
        raise ValueError(f"x: must be a GPU tensor (got device {dev})")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name}: must be on {dev}, the device of x (got {t.device})")


def _at_least(t, n, name):
    """A per-sequence (or per-row) array the kernels read n entries of."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name}: needs at least {n} entries, has {t.numel()}")


def _f32(t, shape, name):
    torch = _torch()
    if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous()):
        raise ValueError(f"{name}: need a contiguous float32 tensor of shape {tuple(shape)}")


def _ref(s):
    return None if s is None else ctypes.byref(s)


def conv1d_fwd_workspace_bytes(rows, C, nseq):
    return int(_lib.load().conv1d_fwd_workspace_bytes(rows, C, nseq))


def conv1d_bwd_workspace_bytes(rows, C):
    return int(_lib.load().conv1d_bwd_workspace_bytes(rows, C))


def conv1d_fwd(x, weight, bias=None, *, cu_seqlens=None, seq_idx=None, seqlen=None, conv_state=None,
               cache_indices=None, has_initial_state=None, history=None, has_history=None, activation="silu",
               out=None, workspace=None, stream=None):
    """y = act(causal depthwise conv of x), packed rows; conv_state is updated in place."""
    torch = _torch()
    lib = _lib.load()
    rows, C = x.shape
    xp, x_ld = _rows2d(x, "x")
    W = _width(weight, C)
    wp, wd = _taps(weight, C, (C, W), "weight")
    bp, bd = _taps(bias, C, (C,), "bias")
    seq, nseq = _seq(rows, cu_seqlens, seq_idx, seqlen)
    pool = _pool(conv_state, cache_indices, has_initial_state, C)
    hist = _hist(history, has_history, C, W)
    _on_gpu(x.device, weight=weight, bias=bias, cu_seqlens=cu_seqlens, seq_idx=seq_idx, conv_state=conv_state,
            cache_indices=cache_indices, has_initial_state=has_initial_state, history=history,
            has_history=has_history, out=out, workspace=workspace)
    _at_least(seq_idx, rows, "seq_idx")
    for t, name in ((cache_indices, "cache_indices"), (has_initial_state, "has_initial_state"),
                    (has_history, "has_history")):
        _at_least(t, max(nseq, 0), name)
    if history is not None and history.shape[0] < max(nseq, 0):
        raise ValueError(f"history: needs a row set for each of the {nseq} sequences")
    if out is None:
        out = torch.empty((rows, C), dtype=torch.bfloat16, device=x.device)
    yp, y_ld = _rows2d(out, "out", C)
    if out.shape[0] != rows:
        raise ValueError("out: must have as many rows as x")
    ws = workspace.data_ptr() if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.conv1d_fwd(xp, rows, C, x_ld, wp, wd, W, bp, bd, ctypes.byref(seq), _ref(pool), _ref(hist),
                        _lib.ACT[activation], yp, y_ld, ws, wsb, _stream(stream, x.device))
    _lib.check(lib, st, "conv1d_fwd")
    return out


def conv1d_state_update(x, weight, bias=None, *, conv_state, cache_indices, activation="silu", out=None,
                        stream=None):
    """One decode token per sequence; conv_state positions 0..2 shift in place."""
    torch = _torch()
    lib = _lib.load()
    nseq, C = x.shape
    xp, x_ld = _rows2d(x, "x")
    wp, wd = _taps(weight, C, (C, 4), "weight")
    bp, bd = _taps(bias, C, (C,), "bias")
    pool = _pool(conv_state, cache_indices, None, C)
    if pool is None:
        raise ValueError("conv_state is required")
    _on_gpu(x.device, weight=weight, bias=bias, conv_state=conv_state, cache_indices=cache_indices, out=out)
    _at_least(cache_indices, nseq, "cache_indices")
    if out is None:
        out = torch.empty((nseq, C), dtype=torch.bfloat16, device=x.device)
    yp, y_ld = _rows2d(out, "out", C)
    if out.shape[0] != nseq:
        raise ValueError("out: must have one row per sequence")
    st = lib.conv1d_state_update(xp, nseq, C, x_ld, wp, wd, bp, bd, ctypes.byref(pool), _lib.ACT[activation],
                                 yp, y_ld, _stream(stream, x.device))
    _lib.check(lib, st, "conv1d_state_update")
    return out


def _tokens3d(t, name, C=None):
    """[nseq, K, C] bf16 with contiguous channels and one uniform row stride across (nseq, K)."""
    if t.dim() != 3 or not _bits_ok(t):
        raise ValueError(f"{name}: need a 3-D bf16 tensor [nseq, K, C]")
    n, K, c = t.shape
    if C is not None and c != C:
        raise ValueError(f"{name}: expected {C} channels")
    if n * K > 0 and c > 1 and t.stride(2) != 1:
        raise ValueError(f"{name}: channels must be contiguous")
    ld = t.stride(1) if K > 1 else (t.stride(0) if n > 1 else c)
    if n > 1 and K > 1 and t.stride(0) != K * t.stride(1):
        raise ValueError(f"{name}: tokens of consecutive sequences must be evenly spaced rows")
    return t.data_ptr(), max(ld, c)


def conv1d_state_update_spec(x, weight, bias=None, *, conv_state, cache_indices, num_accepted=None,
                             activation="silu", out=None, stream=None):
    """K speculative tokens per sequence, x [nseq, K, C]; the history is read at pool positions
    a-1 .. a+1 for num_accepted a (int32 [nseq], None = all 1) and positions 0..K+1 are rewritten
    in place with the last K + 2 raw values."""
    torch = _torch()
    lib = _lib.load()
    nseq, K, C = x.shape
    xp, x_ld = _tokens3d(x, "x")
    wp, wd = _taps(weight, C, (C, 4), "weight")
    bp, bd = _taps(bias, C, (C,), "bias")
    pool = _pool(conv_state, cache_indices, None, C)
    if pool is None:
        raise ValueError("conv_state is required")
    _on_gpu(x.device, weight=weight, bias=bias, conv_state=conv_state, cache_indices=cache_indices,
            num_accepted=num_accepted, out=out)
    _at_least(cache_indices, nseq, "cache_indices")
    _at_least(num_accepted, nseq, "num_accepted")
    if out is None:
        out = torch.empty((nseq, K, C), dtype=torch.bfloat16, device=x.device)
    yp, y_ld = _tokens3d(out, "out", C)
    if tuple(out.shape[:2]) != (nseq, K):
        raise ValueError("out: must have the shape of x")
    acc = _i32(num_accepted, "num_accepted")
    st = lib.conv1d_state_update_spec(xp, nseq, K, C, x_ld, wp, wd, bp, bd, ctypes.byref(pool), acc,
                                      _lib.ACT[activation], yp, y_ld, _stream(stream, x.device))
    _lib.check(lib, st, "conv1d_state_update_spec")
    return out


def conv1d_bwd(x, dy, weight, bias=None, *, cu_seqlens=None, seq_idx=None, seqlen=None, history=None,
               has_history=None, activation="silu", dx=None, dweight=None, want_dbias=None, dbias=None,
               want_dhistory=None, dhistory=None, dtail=None, workspace=None, stream=None):
    """Returns (dx, dweight [C, W] fp32, dbias [C] fp32 or None, dhistory [nseq, W-1, C] or None).

    dtail: bf16 [W-1, C] or None, the next shard's gradient of the last W-1 values of the last
    sequence's extended sequence (its d(history) output there), added into dx (or into that
    sequence's dhistory) before the single rounding."""
    torch = _torch()
    lib = _lib.load()
    rows, C = x.shape
    xp, x_ld = _rows2d(x, "x")
    dyp, dy_ld = _rows2d(dy, "dy", C)
    W = _width(weight, C)
    wp, wd = _taps(weight, C, (C, W), "weight")
    bp, bd = _taps(bias, C, (C,), "bias")
    seq, nseq = _seq(rows, cu_seqlens, seq_idx, seqlen)
    hist = _hist(history, has_history, C, W)
    dev = x.device
    _on_gpu(dev, dy=dy, weight=weight, bias=bias, cu_seqlens=cu_seqlens, seq_idx=seq_idx, history=history,
            has_history=has_history, dx=dx, dweight=dweight, dbias=dbias, dhistory=dhistory, dtail=dtail,
            workspace=workspace)
    if dtail is not None and (tuple(dtail.shape) != (W - 1, C) or not dtail.is_contiguous() or not _bits_ok(dtail)):
        raise ValueError(f"dtail: need a contiguous bf16 tensor of shape {(W - 1, C)}")
    if dy.shape[0] != rows:
        raise ValueError("dy: must have as many rows as x")
    _at_least(seq_idx, rows, "seq_idx")
    _at_least(has_history, max(nseq, 0), "has_history")
    if history is not None and history.shape[0] < max(nseq, 0):
        raise ValueError(f"history: needs a row set for each of the {nseq} sequences")
    _f32(dweight, (C, W), "dweight")
    _f32(dbias, (C,), "dbias")
    if dhistory is not None and (tuple(dhistory.shape) != (max(nseq, 0), W - 1, C) or not dhistory.is_contiguous()
                                 or not _bits_ok(dhistory)):
        raise ValueError(f"dhistory: need a contiguous bf16 tensor of shape {(max(nseq, 0), W - 1, C)}")
    if dx is None:
        dx = torch.empty((rows, C), dtype=torch.bfloat16, device=dev)
    dxp, dx_ld = _rows2d(dx, "dx", C)
    if dx.shape[0] != rows:
        raise ValueError("dx: must have as many rows as x")
    if dweight is None:
        dweight = torch.empty((C, W), dtype=torch.float32, device=dev)
    if want_dbias is None:
        want_dbias = bias is not None or dbias is not None
    if want_dbias and dbias is None:
        dbias = torch.empty((C,), dtype=torch.float32, device=dev)
    if want_dhistory is None:
        want_dhistory = history is not None or dhistory is not None
    if want_dhistory and dhistory is None:
        dhistory = torch.empty((max(nseq, 0), W - 1, C), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        need = lib.conv1d_bwd_workspace_bytes(rows, C)
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    st = lib.conv1d_bwd(xp, dyp, rows, C, x_ld, dy_ld, wp, wd, W, bp, bd, ctypes.byref(seq), _ref(hist),
                        _lib.ACT[activation], dxp, dx_ld, dweight.data_ptr(),
                        None if dbias is None else dbias.data_ptr(),
                        None if dhistory is None else dhistory.data_ptr(),
                        None if dtail is None else dtail.data_ptr(), workspace.data_ptr(), wsb, _stream(stream, dev))
    _lib.check(lib, st, "conv1d_bwd")
    return dx, dweight, (dbias if want_dbias else None), (dhistory if want_dhistory else None)


def conv1d_bwd_noalloc(x, dy, weight, bias=None, *, dx, dweight, dbias=None, dhistory=None, cu_seqlens=None,
                       seq_idx=None, seqlen=None, history=None, has_history=None, dtail=None, activation="silu",
                       stream=None):
    """conv1d_bwd into caller-given outputs with no allocation anywhere: dx bf16 [rows, C] and
    dweight fp32 [C, W] are required; dbias fp32 [C] and dhistory bf16 [nseq, W-1, C] are written
    when given.  The per-range partials use the library's own scratch on the GPU (calls that
    overlap in time on one GPU race on it).  Returns (dx, dweight, dbias, dhistory)."""
    lib = _lib.load()
    rows, C = x.shape
    xp, x_ld = _rows2d(x, "x")
    dyp, dy_ld = _rows2d(dy, "dy", C)
    W = _width(weight, C)
    wp, wd = _taps(weight, C, (C, W), "weight")
    bp, bd = _taps(bias, C, (C,), "bias")
    seq, nseq = _seq(rows, cu_seqlens, seq_idx, seqlen)
    hist = _hist(history, has_history, C, W)
    dev = x.device
    _on_gpu(dev, dy=dy, weight=weight, bias=bias, cu_seqlens=cu_seqlens, seq_idx=seq_idx, history=history,
            has_history=has_history, dx=dx, dweight=dweight, dbias=dbias, dhistory=dhistory, dtail=dtail)
    if dx is None or dweight is None:
        raise ValueError("dx and dweight are required (this entry point allocates nothing)")
    if dtail is not None and (tuple(dtail.shape) != (W - 1, C) or not dtail.is_contiguous() or not _bits_ok(dtail)):
        raise ValueError(f"dtail: need a contiguous bf16 tensor of shape {(W - 1, C)}")
    if dy.shape[0] != rows or dx.shape[0] != rows:
        raise ValueError("dy, dx: must have as many rows as x")
    _at_least(seq_idx, rows, "seq_idx")
    _at_least(has_history, max(nseq, 0), "has_history")
    if history is not None and history.shape[0] < max(nseq, 0):
        raise ValueError(f"history: needs a row set for each of the {nseq} sequences")
    _f32(dweight, (C, W), "dweight")
    _f32(dbias, (C,), "dbias")
    if dhistory is not None and (tuple(dhistory.shape) != (max(nseq, 0), W - 1, C) or not dhistory.is_contiguous()
                                 or not _bits_ok(dhistory)):
        raise ValueError(f"dhistory: need a contiguous bf16 tensor of shape {(max(nseq, 0), W - 1, C)}")
    dxp, dx_ld = _rows2d(dx, "dx", C)
    st = lib.conv1d_bwd_noalloc(xp, dyp, rows, C, x_ld, dy_ld, wp, wd, W, bp, bd, ctypes.byref(seq), _ref(hist),
                                _lib.ACT[activation], dxp, dx_ld, dweight.data_ptr(),
                                None if dbias is None else dbias.data_ptr(),
                                None if dhistory is None else dhistory.data_ptr(),
                                None if dtail is None else dtail.data_ptr(), _stream(stream, dev))
    _lib.check(lib, st, "conv1d_bwd_noalloc")
    return dx, dweight, dbias, dhistory


def conv1d_bwd_combine(dweight_parts, dbias_parts=None, *, dweight=None, dbias=None, stream=None):
    """dweight_parts: fp32 [nshards, C, W] (each shard's dweight, stacked in shard order);
    dbias_parts: fp32 [nshards, C] or None.  Returns (dweight [C, W], dbias [C] or None), each element
    the FP32 sum of its shards in ascending shard order."""
    torch = _torch()
    lib = _lib.load()
    if dweight_parts.dim() != 3 or dweight_parts.dtype != torch.float32 or not dweight_parts.is_contiguous():
        raise ValueError("dweight_parts: need a contiguous float32 tensor [nshards, C, W]")
    S, C, W = dweight_parts.shape
    if dbias_parts is not None and (tuple(dbias_parts.shape) != (S, C) or dbias_parts.dtype != torch.float32
                                    or not dbias_parts.is_contiguous()):
        raise ValueError(f"dbias_parts: need a contiguous float32 tensor of shape {(S, C)}")
    dev = dweight_parts.device
    _on_gpu(dev, dbias_parts=dbias_parts, dweight=dweight, dbias=dbias)
    _f32(dweight, (C, W), "dweight")
    _f32(dbias, (C,), "dbias")
    if dweight is None:
        dweight = torch.empty((C, W), dtype=torch.float32, device=dev)
    if dbias_parts is not None and dbias is None:
        dbias = torch.empty((C,), dtype=torch.float32, device=dev)
    st = lib.conv1d_bwd_combine(dweight_parts.data_ptr(), None if dbias_parts is None else dbias_parts.data_ptr(),
                                S, C, W, dweight.data_ptr(), None if dbias_parts is None else dbias.data_ptr(),
                                _stream(stream, dev))
    _lib.check(lib, st, "conv1d_bwd_combine")
    return dweight, (dbias if dbias_parts is not None else None)


# ------------------------------------------------------------------ channels-first [B, D, T]
def _cf3d(t, name, shape=None):
    if t.dim() != 3 or not _bits_ok(t):
        raise ValueError(f"{name}: need a 3-D bf16 tensor [B, D, T]")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError(f"{name}: the time axis must be contiguous")
    return t.data_ptr(), t.stride(0), t.stride(1)


def conv1d_bwd_cf_workspace_bytes(B, D):
    return int(_lib.load().conv1d_bwd_cf_workspace_bytes(B, D))


def conv1d_fwd_cf(x, weight, bias=None, *, activation="silu", out=None, stream=None):
    """y = act(causal width-W conv along T) for x [B, D, T]; every (b, d) row is one sequence."""
    torch = _torch()
    lib = _lib.load()
    B, D, T = x.shape
    xp, xsb, xsd = _cf3d(x, "x")
    W = _width(weight, D)
    wp, wd = _taps(weight, D, (D, W), "weight")
    bp, bd = _taps(bias, D, (D,), "bias")
    _on_gpu(x.device, weight=weight, bias=bias, out=out)
    if out is None:
        out = torch.empty((B, D, T), dtype=torch.bfloat16, device=x.device)
    yp, ysb, ysd = _cf3d(out, "out", (B, D, T))
    st = lib.conv1d_fwd_cf(xp, B, D, T, xsb, xsd, wp, wd, W, bp, bd, _lib.ACT[activation], yp, ysb, ysd,
                           _stream(stream, x.device))
    _lib.check(lib, st, "conv1d_fwd_cf")
    return out


def conv1d_bwd_cf(x, dy, weight, bias=None, *, activation="silu", dx=None, dweight=None, want_dbias=None,
                  dbias=None, workspace=None, stream=None):
    """(dx [B, D, T], dweight [D, W] fp32, dbias [D] fp32 or None) for the channels-first layout."""
    torch = _torch()
    lib = _lib.load()
    B, D, T = x.shape
    xp, xsb, xsd = _cf3d(x, "x")
    dyp, dysb, dysd = _cf3d(dy, "dy", (B, D, T))
    W = _width(weight, D)
    wp, wd = _taps(weight, D, (D, W), "weight")
    bp, bd = _taps(bias, D, (D,), "bias")
    dev = x.device
    _on_gpu(dev, dy=dy, weight=weight, bias=bias, dx=dx, dweight=dweight, dbias=dbias, workspace=workspace)
    _f32(dweight, (D, W), "dweight")
    _f32(dbias, (D,), "dbias")
    if dx is None:
        dx = torch.empty((B, D, T), dtype=torch.bfloat16, device=dev)
    dxp, dxsb, dxsd = _cf3d(dx, "dx", (B, D, T))
    if dweight is None:
        dweight = torch.empty((D, W), dtype=torch.float32, device=dev)
    if want_dbias is None:
        want_dbias = bias is not None
    if want_dbias and dbias is None:
        dbias = torch.empty((D,), dtype=torch.float32, device=dev)
    need = lib.conv1d_bwd_cf_workspace_bytes(B, D)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    st = lib.conv1d_bwd_cf(xp, dyp, B, D, T, xsb, xsd, dysb, dysd, wp, wd, W, bp, bd, _lib.ACT[activation], dxp,
                           dxsb, dxsd, dweight.data_ptr(), dbias.data_ptr() if want_dbias else None,
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream, dev))
    _lib.check(lib, st, "conv1d_bwd_cf")
    return dx, dweight, (dbias if want_dbias else None)
