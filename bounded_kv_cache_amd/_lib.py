"""ctypes view of libprefix_sliding.so (the C ABI declared in include/prefix_sliding.h).

Loading never falls back to anything: if the built library is missing the
import of the binding raises, naming the build step."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libprefix_sliding.so")

PS_OK, PS_INVALID_ARGUMENT, PS_UNSUPPORTED, PS_WORKSPACE_TOO_SMALL, PS_HIP_ERROR = range(5)
PS_BF16, PS_F32 = 0, 1
PS_PE_CONTINUE, PS_PE_RESET, PS_PE_RESET_RECOMPUTE = 0, 1, 2


class AttnDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("pe_mode", ctypes.c_int32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("page_size", ctypes.c_int32), ("slot_capacity", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int64)]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_pA = ctypes.POINTER(AttnDesc)
_pC = ctypes.POINTER(CacheDesc)

SIGNATURES = {
    "ps_kv_append": (_i32, [_pA, _pC, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp]),
    "ps_decode_attn": (_i32, [_pA, _pC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _sz, _vp]),
    "ps_decode_step": (_i32, [_pA, _pC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _sz, _vp]),
    "ps_decode_step_noalloc": (_i32, [_pA, _pC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp]),
    "ps_decode_noalloc_scratch_bytes": (_sz, []),
    "ps_decode_num_splits": (_i32, [_pA, _pC, _i32]),
    "ps_decode_workspace_size": (_sz, [_pA, _pC, _i32, _i32]),
    "ps_prefill_attn": (_i32, [_pA, _i32, _i32, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "ps_prefill_workspace_size": (_sz, [_pA, _i32, _i32, _i32]),
    "ps_chunk_prefill_attn": (_i32, [_pA, _pC, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                                     _sz, _vp]),
    "ps_chunk_prefill_workspace_size": (_sz, [_pA, _pC, _i32, _i32]),
    "ps_prefill_attn_backward": (_i32, [_pA, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp,
                                        _vp, _vp, _vp, _sz, _vp]),
    "ps_prefill_backward_workspace_size": (_sz, [_pA, _i32, _i32, _i32]),
    "ps_prefill_backward_ds_workspace_size": (_sz, [_pA, _i32, _i32, _i64, _i32, _i32, _i32]),
    "ps_heavy_decode_step": (_i32, [_pA, _pC, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                    _i32, _vp, _sz, _vp]),
    "ps_heavy_workspace_size": (_sz, [_pA, _pC, _i32, _i32]),
    "ps_prefill_tile_shape": (_i32, [_pA, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "ps_prefill_plan": (_i32, [_pA, _i32, _i32, _i64, _i32, _i32, _vp, _i32, _vp, _vp]),
    "ps_read_probe": (_i32, [_vp, _sz, _vp, _vp]),
    "ps_last_error": (ctypes.c_char_p, []),
    "ps_status_string": (ctypes.c_char_p, [_i32]),
    "ps_abi_version": (_i32, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class PSError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{load().ps_status_string(status).decode()}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != PS_OK:
        raise PSError(status, load().ps_last_error().decode())
