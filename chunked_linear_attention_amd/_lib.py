"""ctypes loader for libttt_mi355x.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libttt_mi355x.so")

TTT_OK = 0
TTT_EINVAL = -1
TTT_EUNSUPPORTED = -2
TTT_EWORKSPACE = -3
TTT_EHIP = -4

EXPORTS = ("ttt_status_string", "ttt_abi_version", "ttt_linear_workspace_bytes", "ttt_linear_fwd",
           "ttt_linear_workspace_bytes_seg", "ttt_linear_fwd_seg",
           "lact_swiglu_workspace_bytes", "lact_swiglu_fwd", "ttt_linear_decode",
           "lact_swiglu_decode_workspace_bytes", "lact_swiglu_decode",
           "lact_swiglu_rule_workspace_bytes", "lact_swiglu_fwd_rule", "window_attention_fwd",
           "ttt_linear_bwd_workspace_bytes", "ttt_linear_bwd", "ttt_probe_mfma_bf16", "ttt_probe_gemm_bf16",
           "ttt_linear_noalloc_max_scratch_bytes", "ttt_linear_fwd_noalloc",
           "lact_swiglu_bwd_workspace_bytes", "lact_swiglu_bwd")

_lock = threading.Lock()
_lib = None


class TTTError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)} ({status})")


def load() -> ctypes.CDLL:
    """Load the HIP library; raise if it has not been built (there is no fallback)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python chunked_linear_attention_amd/build.py`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.ttt_status_string.argtypes = [i]
        lib.ttt_status_string.restype = ctypes.c_char_p
        lib.ttt_abi_version.argtypes = []
        lib.ttt_abi_version.restype = i
        lib.ttt_linear_workspace_bytes.argtypes = [i] * 9
        lib.ttt_linear_workspace_bytes.restype = sz
        lib.ttt_linear_fwd.argtypes = [vp, vp, vp, i, vp, vp, vp, vp] + [i] * 8 + [vp, sz, vp]
        lib.ttt_linear_fwd.restype = i
        lib.ttt_linear_workspace_bytes_seg.argtypes = [i] * 10
        lib.ttt_linear_workspace_bytes_seg.restype = sz
        lib.ttt_linear_fwd_seg.argtypes = [vp, vp, vp, i, vp, vp, vp, vp] + [i] * 9 + [vp, sz, vp]
        lib.ttt_linear_fwd_seg.restype = i
        lib.lact_swiglu_workspace_bytes.argtypes = [i] * 10
        lib.lact_swiglu_workspace_bytes.restype = sz
        lib.lact_swiglu_fwd.argtypes = [vp, vp, vp, i, vp, vp, vp, vp, vp, vp, vp, vp] + [i] * 10 + \
            [vp, sz, vp, vp]
        lib.lact_swiglu_fwd.restype = i
        f = ctypes.c_float
        lib.lact_swiglu_rule_workspace_bytes.argtypes = [i] * 11
        lib.lact_swiglu_rule_workspace_bytes.restype = sz
        lib.lact_swiglu_fwd_rule.argtypes = [vp, vp, vp, i, vp, vp, vp, vp, vp, vp, vp, vp] + \
            [i] * 11 + [f, i, f, vp, vp, vp, vp, sz, vp, vp]
        lib.lact_swiglu_fwd_rule.restype = i
        lib.ttt_linear_bwd_workspace_bytes.argtypes = [i] * 9
        lib.ttt_linear_bwd_workspace_bytes.restype = sz
        lib.ttt_linear_bwd.argtypes = [vp, vp, vp, i, vp, vp, vp, vp, vp, vp, vp, vp, vp] + \
            [i] * 8 + [vp, sz, vp]
        lib.ttt_linear_bwd.restype = i
        lib.window_attention_fwd.argtypes = [vp, vp, vp, i, vp, i, i, i, i, i, f, i, vp]
        lib.window_attention_fwd.restype = i
        lib.ttt_linear_decode.argtypes = [vp, vp, vp, i, vp, vp, vp, i, vp, i, i, i, i, vp]
        lib.ttt_linear_decode.restype = i
        lib.lact_swiglu_decode_workspace_bytes.argtypes = [i] * 5
        lib.lact_swiglu_decode_workspace_bytes.restype = sz
        lib.lact_swiglu_decode.argtypes = [vp, i, vp, vp, vp, vp, i, i, i, i, vp, sz, vp]
        lib.lact_swiglu_decode.restype = i
        lib.ttt_probe_mfma_bf16.argtypes = [vp, i, i, vp]
        lib.ttt_probe_mfma_bf16.restype = i
        lib.ttt_probe_gemm_bf16.argtypes = [vp, vp, vp] + [i] * 7 + [vp]
        lib.ttt_probe_gemm_bf16.restype = i
        lib.ttt_linear_noalloc_max_scratch_bytes.argtypes = []
        lib.ttt_linear_noalloc_max_scratch_bytes.restype = sz
        lib.ttt_linear_fwd_noalloc.argtypes = [vp, vp, vp, i, vp, vp, vp, vp] + [i] * 8 + [vp]
        lib.ttt_linear_fwd_noalloc.restype = i
        lib.lact_swiglu_bwd_workspace_bytes.argtypes = [i] * 10
        lib.lact_swiglu_bwd_workspace_bytes.restype = sz
        lib.lact_swiglu_bwd.argtypes = [vp, vp, vp, i] + [vp] * 15 + [i] * 10 + [vp, sz, vp]
        lib.lact_swiglu_bwd.restype = i
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().ttt_status_string(int(status)).decode()
