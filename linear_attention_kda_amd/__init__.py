"""Kimi Delta Attention (KDA) on MI355X (gfx950): chunked prefill and decode.

The computation runs in hand-written HIP kernels behind the C ABI declared
in ``include/kda.h`` (library ``libkda.so`` in this directory).  This package
is the thin Python binding over that ABI; torch supplies device memory and
streams.  The library is loaded on first use of a binding name; if it is
missing that raises ImportError (there is no fallback).
"""
_BINDING_NAMES = ("EXPORTED", "GATES", "KDA_BF16", "KDA_F32", "KDA_GATE_CHANNEL", "KDA_GATE_LOG_CHANNEL",
                  "KDA_GATE_LOG_SCALAR", "KDA_GATE_NONE",
                  "KDA_GATE_SCALAR", "KDA_GATE_SOFTPLUS_CHANNEL", "KDA_GATE_SOFTPLUS_SCALAR",
                  "KDA_ACT_QK_SILU_L2NORM", "KDA_ACT_BETA_SIGMOID", "LIB_PATH", "KdaError", "chunk_fwd", "chunk_fwd_workspace_size",
                  "decode_step", "decode_tokens", "lib", "set_validation", "set_schedule", "status_string",
                  "KDA_SCHEDULE_AUTO", "KDA_SCHEDULE_TWO_PHASE", "KDA_SCHEDULE_OVERLAP", "KDA_SCHEDULE_SPLIT",
                  "SCHEDULES",
                  "KDA_ERR_INVALID_VALUE", "KDA_ERR_STREAM_CAPTURE", "KDA_SCHED_ERR_TIMEOUT", "KDA_SCHED_ERR_XCD",
                  "chunk_fwd_status", "release", "validation_enabled", "set_sched_wait_limit",
                  "chunk_fwd_noalloc", "KDA_ERR_TOO_LARGE", "NOALLOC_SCRATCH_BYTES")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)


__all__ = list(_BINDING_NAMES)
