"""ctypes view of the C ABI declared in include/conv1d.h (argument marshalling only)."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcausal_conv1d.so")

c_p = ctypes.c_void_p
c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_size = ctypes.c_size_t

OK, EINVAL, EWORKSPACE, EUNSUPPORTED, EHIP, ETOOLARGE = 0, 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 20 << 20  # CONV1D_NOALLOC_SCRATCH_BYTES
BF16, F32 = 0, 1
ACT = {"none": 0, None: 0, "silu": 1, "swish": 1}


class Seq(ctypes.Structure):
    _fields_ = [("cu_seqlens", c_p), ("nseq", c_i64), ("seq_idx", c_p), ("seqlen", c_i64)]


class Pool(ctypes.Structure):
    _fields_ = [("ptr", c_p), ("slots", c_i64), ("len", c_i64), ("s_slot", c_i64), ("s_chan", c_i64),
                ("s_pos", c_i64), ("cache_indices", c_p), ("has_initial_state", c_p)]


class Hist(ctypes.Structure):
    _fields_ = [("ptr", c_p), ("has_history", c_p)]


# name -> (restype, argtypes); must match include/conv1d.h
SIGNATURES = {
    "conv1d_fwd": (c_int, [c_p, c_i64, c_i64, c_i64, c_p, c_int, c_int, c_p, c_int, ctypes.POINTER(Seq),
                           ctypes.POINTER(Pool), ctypes.POINTER(Hist), c_int, c_p, c_i64, c_p, c_size, c_p]),
    "conv1d_state_update": (c_int, [c_p, c_i64, c_i64, c_i64, c_p, c_int, c_p, c_int, ctypes.POINTER(Pool),
                                    c_int, c_p, c_i64, c_p]),
    "conv1d_state_update_spec": (c_int, [c_p, c_i64, c_i64, c_i64, c_i64, c_p, c_int, c_p, c_int,
                                         ctypes.POINTER(Pool), c_p, c_int, c_p, c_i64, c_p]),
    "conv1d_bwd": (c_int, [c_p, c_p, c_i64, c_i64, c_i64, c_i64, c_p, c_int, c_int, c_p, c_int, ctypes.POINTER(Seq),
                           ctypes.POINTER(Hist), c_int, c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_size, c_p]),
    "conv1d_bwd_combine": (c_int, [c_p, c_p, c_i64, c_i64, c_int, c_p, c_p, c_p]),
    "conv1d_bwd_noalloc": (c_int, [c_p, c_p, c_i64, c_i64, c_i64, c_i64, c_p, c_int, c_int, c_p, c_int,
                                   ctypes.POINTER(Seq), ctypes.POINTER(Hist), c_int, c_p, c_i64, c_p, c_p, c_p, c_p,
                                   c_p]),
    "conv1d_fwd_cf": (c_int, [c_p, c_i64, c_i64, c_i64, c_i64, c_i64, c_p, c_int, c_int, c_p, c_int, c_int, c_p, c_i64,
                              c_i64, c_p]),
    "conv1d_bwd_cf": (c_int, [c_p, c_p, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_p, c_int, c_int, c_p, c_int,
                              c_int, c_p, c_i64, c_i64, c_p, c_p, c_p, c_size, c_p]),
    "conv1d_bwd_cf_workspace_bytes": (c_size, [c_i64, c_i64]),
    "conv1d_fwd_workspace_bytes": (c_size, [c_i64, c_i64, c_i64]),
    "conv1d_bwd_workspace_bytes": (c_size, [c_i64, c_i64]),
    "conv1d_status_str": (ctypes.c_char_p, [c_int]),
}

_LIB = None


def load(path=LIB_PATH):
    """Load the HIP library (built by ``python -m causal_depthwise_conv1d_width_amd.build``).

    Raises ImportError when it is missing: there is no fallback implementation."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m causal_depthwise_conv1d_width_amd.build` "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _LIB = lib
    return lib


class Conv1dError(RuntimeError):
    pass


def check(lib, status, what):
    if status == OK:
        return
    msg = f"{what}: {lib.conv1d_status_str(status).decode()} (status {status})"
    if status == EINVAL:
        raise ValueError(msg)
    raise Conv1dError(msg)
