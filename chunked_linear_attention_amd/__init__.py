"""MI355X-native TTT-layer forward (TTT-Linear and LaCT SwiGLU).

The compute lives in libttt_mi355x.so (hand-written gfx950 HIP kernels behind
a C ABI, declared in include/ttt.h).  This package is a thin binding: it
checks tensors, allocates outputs and the workspace with torch (device memory
and the current stream only) and calls the library.  Nothing here computes.
"""
from .ops import (CAUSAL, NONCAUSAL, LOSS_DOT, LOSS_MSE, RULE_GD, RULE_MOMENTUM, RULE_MUON,
                  lact_swiglu_bwd, lact_swiglu_decode, lact_swiglu_decode_workspace_bytes,
                  lact_swiglu_fwd,
                  lact_swiglu_fwd_rule, lact_swiglu_rule_workspace_bytes,
                  lact_swiglu_workspace_bytes, ttt_linear_bwd, ttt_linear_decode, ttt_linear_fwd,
                  ttt_linear_workspace_bytes, window_attention_fwd)
from ._lib import TTTError, load as load_library, status_string

__all__ = ["ttt_linear_fwd", "lact_swiglu_fwd", "ttt_linear_workspace_bytes",
           "lact_swiglu_workspace_bytes", "ttt_linear_decode", "lact_swiglu_decode",
           "lact_swiglu_decode_workspace_bytes", "lact_swiglu_fwd_rule",
           "lact_swiglu_rule_workspace_bytes", "window_attention_fwd", "ttt_linear_bwd",
           "lact_swiglu_bwd", "RULE_GD", "RULE_MOMENTUM", "RULE_MUON", "TTTError", "load_library",
           "status_string",
           "CAUSAL", "NONCAUSAL", "LOSS_DOT", "LOSS_MSE"]
