"""ctypes binding of ``libkda.so`` (C ABI in ``include/kda.h``).

Argument marshalling only: shapes and dtypes are checked, outputs and the
workspace are allocated with torch on the inputs' device, and raw device
pointers plus torch's current HIP stream are handed to the library.  Every
step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing the import fails loudly.
"""
from __future__ import annotations

import atexit
import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY loads another build of the same ABI (the CPU sanitizer job's
# host-only build of the argument checks); by default the in-tree library
LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(PKG_DIR, "libkda.so")

KDA_F32 = 0
KDA_BF16 = 1

# forget-gate forms (kda_gate): one gate per key channel, one per token and
# head shared by all channels, or none
KDA_GATE_CHANNEL = 0
KDA_GATE_SCALAR = 1
KDA_GATE_NONE = 2
KDA_GATE_LOG_CHANNEL = 3
KDA_GATE_LOG_SCALAR = 4
KDA_GATE_SOFTPLUS_CHANNEL = 5
KDA_GATE_SOFTPLUS_SCALAR = 6
GATES = {"channel": KDA_GATE_CHANNEL, "scalar": KDA_GATE_SCALAR, "none": KDA_GATE_NONE,
         "log_channel": KDA_GATE_LOG_CHANNEL, "log_scalar": KDA_GATE_LOG_SCALAR,
         "softplus_channel": KDA_GATE_SOFTPLUS_CHANNEL, "softplus_scalar": KDA_GATE_SOFTPLUS_SCALAR}
_PER_CHANNEL = (KDA_GATE_CHANNEL, KDA_GATE_LOG_CHANNEL, KDA_GATE_SOFTPLUS_CHANNEL)
_PER_TOKEN = (KDA_GATE_SCALAR, KDA_GATE_LOG_SCALAR, KDA_GATE_SOFTPLUS_SCALAR)
# input activations (kda_input_act flags)
KDA_ACT_QK_SILU_L2NORM = 1
KDA_ACT_BETA_SIGMOID = 2
# prefill schedules (kda_schedule)
KDA_SCHEDULE_AUTO = 0
KDA_SCHEDULE_TWO_PHASE = 1
KDA_SCHEDULE_OVERLAP = 2
KDA_SCHEDULE_SPLIT = 3
SCHEDULES = {"auto": KDA_SCHEDULE_AUTO, "two_phase": KDA_SCHEDULE_TWO_PHASE, "overlap": KDA_SCHEDULE_OVERLAP,
             "split": KDA_SCHEDULE_SPLIT}

# error bits of kda_chunk_fwd_status
KDA_SCHED_ERR_TIMEOUT = 1
KDA_SCHED_ERR_XCD = 2

# names exported by include/kda.h
EXPORTED = ("kda_status_string", "kda_set_validation", "kda_set_schedule", "kda_chunk_fwd_status",
            "kda_release", "kda_set_sched_wait_limit", "kda_chunk_fwd_workspace_size", "kda_chunk_fwd",
            "kda_chunk_fwd_gated", "kda_chunk_fwd_ex", "kda_decode_step", "kda_decode_step_gated",
            "kda_decode_tokens", "kda_decode_tokens_ex", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_module",
            "kda_decode_tokens_module")
KDA_ERR_INVALID_VALUE = 11
KDA_ERR_STREAM_CAPTURE = 13
KDA_ERR_TOO_LARGE = 14
NOALLOC_SCRATCH_BYTES = 64 << 20   # the static device scratch of kda_chunk_fwd_noalloc


class KdaModuleOps(ctypes.Structure):
    """kda_module_ops: device pointers (None: operation off) and the norm's eps."""
    _fields_ = [("conv_q", ctypes.c_void_p), ("conv_k", ctypes.c_void_p), ("conv_v", ctypes.c_void_p),
                ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float), ("out_gate", ctypes.c_void_p),
                ("conv_state", ctypes.c_void_p)]


class KdaError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, where: str, status: int):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i32]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                  f32, i32, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd_gated.restype = i32
    lib.kda_chunk_fwd_gated.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                        f32, i32, vp, vp, vp, sz, vp]
    lib.kda_decode_step.restype = i32
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.kda_decode_step_gated.restype = i32
    lib.kda_decode_step_gated.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.kda_decode_tokens.restype = i32
    lib.kda_decode_tokens.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                      vp, vp]
    lib.kda_chunk_fwd_ex.restype = i32
    lib.kda_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_uint, vp, vp, i32, i32, i32, i32, i32,
                                     i32, f32, i32, vp, vp, vp, sz, vp]
    lib.kda_decode_tokens_ex.restype = i32
    lib.kda_decode_tokens_ex.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_uint, vp, vp, i32, i32, i32, i32,
                                         i32, f32, i32, vp, vp]
    lib.kda_set_validation.restype = i32
    lib.kda_set_validation.argtypes = [i32]
    lib.kda_set_schedule.restype = i32
    lib.kda_set_schedule.argtypes = [i32]
    lib.kda_chunk_fwd_status.restype = i32
    lib.kda_chunk_fwd_status.argtypes = [vp, vp, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_uint)]
    lib.kda_chunk_fwd_noalloc.restype = i32
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_uint, vp, vp, i32, i32, i32, i32, i32,
                                          i32, f32, i32, vp, vp, vp]
    lib.kda_chunk_fwd_module.restype = i32
    lib.kda_chunk_fwd_module.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_uint, ctypes.POINTER(KdaModuleOps), vp,
                                         vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, sz, vp]
    lib.kda_decode_tokens_module.restype = i32
    lib.kda_decode_tokens_module.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_uint, ctypes.POINTER(KdaModuleOps),
                                             vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.kda_release.restype = None
    lib.kda_release.argtypes = []
    lib.kda_set_sched_wait_limit.restype = ctypes.c_longlong
    lib.kda_set_sched_wait_limit.argtypes = [ctypes.c_longlong]
    return lib


lib = _load()
# the overlapped schedule's internal streams go before the interpreter (and
# the HIP runtime under it) shuts down
atexit.register(lib.kda_release)


def status_string(status: int) -> str:
    return lib.kda_status_string(int(status)).decode()


def set_validation(enable: bool) -> bool:
    """Turn the library's device-side value checks on or off (process-wide);
    returns the previous setting.  While on, every call synchronises its
    stream and raises KdaError (status KDA_ERR_INVALID_VALUE) on inputs
    outside the method's domain."""
    return bool(lib.kda_set_validation(1 if enable else 0))


def validation_enabled() -> bool:
    return bool(lib.kda_set_validation(-1))


def chunk_fwd_status(workspace, stream=None):
    """(schedule name, error bits) of the last chunk_fwd call that launched
    work with this workspace tensor (see kda_chunk_fwd_status; synchronises
    the stream)."""
    sched, errs = ctypes.c_int(0), ctypes.c_uint(0)
    st = lib.kda_chunk_fwd_status(_ptr(workspace), stream if stream is not None else _stream(workspace.device),
                                  ctypes.byref(sched), ctypes.byref(errs))
    if st != 0:
        raise KdaError("kda_chunk_fwd_status", st)
    names = {v: k for k, v in SCHEDULES.items()}
    return names.get(sched.value, str(sched.value)), int(errs.value)


def set_sched_wait_limit(ticks: int) -> int:
    """Bound on one ready-flag wait of the overlapped scan, in 100 MHz ticks
    (kda_set_sched_wait_limit; 0 gives up at once).  Returns the previous."""
    return int(lib.kda_set_sched_wait_limit(int(ticks)))


def release() -> None:
    """Destroy the library's internal streams and events (kda_release)."""
    lib.kda_release()


def set_schedule(schedule: str) -> str:
    """Choose how chunk_fwd schedules its kernels: "auto", "two_phase" or
    "overlap" (process-wide; see kda_set_schedule); returns the previous
    setting's name."""
    if schedule not in SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(SCHEDULES)}")
    prev = lib.kda_set_schedule(SCHEDULES[schedule])
    return {v: k for k, v in SCHEDULES.items()}[prev]


def chunk_fwd_workspace_size(B: int, T: int, H: int, d_k: int, d_v: int, N: int = -1,
                             dtype: int = KDA_BF16) -> int:
    return int(lib.kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, N, dtype))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _prep(t):
    """Contiguous and 16-byte aligned (the ABI's layout contract); a view that
    starts mid-allocation at an unaligned address is copied."""
    if t is None:
        return None
    t = t.contiguous()
    if t.data_ptr() % 16:
        t = t.clone()
    return t


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _gate_code(gate, alpha, q):
    """kda_gate code: given by name, else read from alpha's shape (which
    cannot tell a log gate from a gate: the log forms are named)."""
    if gate is None:
        if alpha is None:
            return KDA_GATE_NONE
        return KDA_GATE_SCALAR if alpha.dim() == q.dim() - 1 else KDA_GATE_CHANNEL
    if gate not in GATES:
        raise ValueError(f"gate must be one of {sorted(GATES)}, got {gate!r}")
    return GATES[gate]


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _module_ops(torch, H, d_k, d_v, dtype, n_out, conv, norm_weight, norm_eps, out_gate, conv_state, n_state):
    """kda_module_ops from tensors (None: off), checked for dtype and size;
    returns (ops, tensors to keep alive during the call)."""
    wq, wk, wv = map(_prep, conv) if conv is not None else (None, None, None)
    for w, d in ((wq, d_k), (wk, d_k), (wv, d_v)):
        if w is not None and (w.dtype != torch.float32 or w.numel() != H * d * 4):
            raise ValueError("convolution taps must be float32 [H, d, 4]")
    norm_weight = _prep(norm_weight)
    if norm_weight is not None and (norm_weight.dtype != torch.float32 or norm_weight.numel() != d_v):
        raise ValueError("norm_weight must be float32 [d_v]")
    out_gate = _prep(out_gate)
    if out_gate is not None and (out_gate.dtype != dtype or out_gate.numel() != n_out):
        raise ValueError("out_gate must have the dtype and size of the output")
    if conv_state is not None:
        if (not conv_state.is_contiguous() or conv_state.dtype != dtype or conv_state.data_ptr() % 16
                or conv_state.numel() != n_state * 3 * (2 * d_k + d_v)):
            raise ValueError("conv_state must be a contiguous, 16-byte aligned [N, H, 3, 2 d_k + d_v] tensor "
                             "of the inputs' dtype")
    ops = KdaModuleOps(_ptr(wq), _ptr(wk), _ptr(wv), _ptr(norm_weight), float(norm_eps), _ptr(out_gate),
                       _ptr(conv_state))
    return ops, (wq, wk, wv, norm_weight, out_gate, conv_state)


def chunk_fwd_noalloc(q, k, v, alpha, beta, S0=None, cu_seqlens=None, scale=None, *, gate=None, out=None,
                      S_final=None, act=0):
    """chunk_fwd through kda_chunk_fwd_noalloc: no workspace, the library's
    static device scratch instead (outputs are still allocated here unless
    given: pass ``out`` and ``S_final`` to allocate nothing)."""
    return chunk_fwd(q, k, v, alpha, beta, S0, cu_seqlens, scale, gate=gate, out=out, S_final=S_final, act=act,
                     _noalloc=True)


def chunk_fwd(q, k, v, alpha, beta, S0=None, cu_seqlens=None, scale=None, *, gate=None, out=None,
              S_final=None, workspace=None, act=0, conv=None, norm_weight=None, norm_eps=1e-6, out_gate=None,
              conv_state=None, _noalloc=False):
    """Chunked prefill.  Returns (o, S_final).

    ``act``: kda_input_act flags (KDA_ACT_QK_SILU_L2NORM, KDA_ACT_BETA_SIGMOID)
    applied to the raw q, k and beta as the kernels load them.
    Module operations (kda_module_ops; any given selects
    kda_chunk_fwd_module): ``conv`` = (w_q, w_k, w_v), fp32 taps [H, d_k, 4],
    [H, d_k, 4], [H, d_v, 4] of the short causal convolution (needs
    KDA_ACT_QK_SILU_L2NORM in ``act``); ``norm_weight`` [d_v] fp32 gains of the
    output RMS norm (with ``norm_eps``); ``out_gate`` logits of the output gate,
    shaped and typed like the output; ``conv_state`` (with ``conv``) an
    [N, H, 3, 2 d_k + d_v] tensor of the inputs' dtype that receives each
    sequence's last three raw tokens, for decode_tokens to continue from.
    Dense batch: q, k [B, T, H, d_k]; v [B, T, H, d_v]; beta [B, T, H].
    alpha: [B, T, H, d_k] (gate "channel"), [B, T, H] (gate "scalar"), or
    None (gate "none"); ``gate`` defaults to what alpha's shape says.
    Packed batch: pass ``cu_seqlens`` (int32, device, N+1 offsets) and tensors
    with a packed token axis, [T, H, d] or [1, T, H, d].
    S0: [N, H, d_v, d_k] fp32 or None.  ``S_final`` may be ``S0`` (in place).
    """
    import torch
    dt = _dtype_code(q)
    gc = _gate_code(gate, alpha, q)
    if gc == KDA_GATE_NONE:
        alpha = None
    q, k, v, alpha, beta = map(_prep, (q, k, v, alpha, beta))
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if (alpha is not None and alpha.dtype != torch.float32) or beta.dtype != torch.float32:
        raise TypeError("alpha and beta must be float32")
    d_k, d_v, H = q.shape[-1], v.shape[-1], q.shape[-2]
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        cu_seqlens = _prep(cu_seqlens)
        B, T = 1, q.numel() // (H * d_k)
        N = cu_seqlens.numel() - 1
    else:
        if q.dim() != 4:
            raise ValueError("dense q must be [B, T, H, d_k]")
        B, T = q.shape[0], q.shape[1]
        N = B
    if k.shape != q.shape:
        raise ValueError("k must have the shape of q")
    if gc in _PER_CHANNEL and alpha.shape != q.shape:
        raise ValueError("per-channel alpha must have the shape of q")
    if gc in _PER_TOKEN and alpha.numel() != B * T * H:
        raise ValueError("scalar alpha must have one value per token and head")
    if v.numel() != B * T * H * d_v or beta.numel() != B * T * H:
        raise ValueError("v / beta sizes do not match q")
    if S0 is not None:
        if S0.dtype != torch.float32:
            raise TypeError("S0 must be float32")
        S0 = _prep(S0)
        if S0.numel() != N * H * d_v * d_k:
            raise ValueError("S0 must be [N, H, d_v, d_k]")
    dev = q.device
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if S_final is None:
        S_final = torch.empty((N, H, d_v, d_k), dtype=torch.float32, device=dev)
    if _noalloc:
        st = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), gc, _ptr(beta), int(act), _ptr(S0),
                                       _ptr(cu_seqlens), N, B, T, H, d_k, d_v, float(scale) if scale else 0.0, dt,
                                       _ptr(out), _ptr(S_final), _stream(dev))
        if st != 0:
            raise KdaError("kda_chunk_fwd_noalloc", st)
        return out, S_final
    ws_need = chunk_fwd_workspace_size(B, T, H, d_k, d_v, N if cu_seqlens is not None else -1, dt)
    if workspace is None or workspace.numel() < ws_need:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=dev)
    if conv is not None or norm_weight is not None or out_gate is not None:
        ops, _keep = _module_ops(torch, H, d_k, d_v, v.dtype, v.numel(), conv, norm_weight, norm_eps, out_gate,
                                 conv_state, N * H)
        st = lib.kda_chunk_fwd_module(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), gc, _ptr(beta), int(act),
                                      ctypes.byref(ops), _ptr(S0), _ptr(cu_seqlens), N, B, T, H, d_k, d_v,
                                      float(scale) if scale else 0.0, dt, _ptr(out), _ptr(S_final),
                                      _ptr(workspace), workspace.numel(), _stream(dev))
        if st != 0:
            raise KdaError("kda_chunk_fwd_module", st)
    else:
        st = lib.kda_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), gc, _ptr(beta), int(act), _ptr(S0),
                                  _ptr(cu_seqlens), N, B, T, H, d_k, d_v,
                                  float(scale) if scale else 0.0, dt, _ptr(out), _ptr(S_final),
                                  _ptr(workspace), workspace.numel(), _stream(dev))
        if st != 0:
            raise KdaError("kda_chunk_fwd_ex", st)
    if validation_enabled():
        # with value checks on the call has already waited for the device;
        # a schedule error (a record wait that gave up) means wrong results
        sched, errs = chunk_fwd_status(workspace)
        if errs:
            raise RuntimeError(f"kda_chunk_fwd: the {sched} schedule reported error bits {errs:#x} "
                               "(results are wrong)")
    return out, S_final


def decode_step(q, k, v, alpha, beta, S, scale=None, *, gate=None, out=None, act=0):
    """One token for N sequences: q, k [N, H, d_k]; v [N, H, d_v]; beta [N, H];
    alpha [N, H, d_k] (gate "channel"), [N, H] ("scalar") or None ("none");
    S [N, H, d_v, d_k] fp32, updated in place.  Returns o.  With input
    activations (``act``) the step runs as one token of decode_tokens."""
    import torch
    if act:
        o, _ = decode_tokens(q.unsqueeze(1), k.unsqueeze(1), v.unsqueeze(1),
                             None if alpha is None else alpha.unsqueeze(1), beta.unsqueeze(1), S, S_out=S,
                             scale=scale, gate=gate, act=act,
                             out=None if out is None else out.unsqueeze(1))
        return o.squeeze(1)
    dt = _dtype_code(q)
    gc = _gate_code(gate, alpha, q)
    if gc == KDA_GATE_NONE:
        alpha = None
    if not S.is_contiguous() or S.dtype != torch.float32 or S.data_ptr() % 16:
        raise ValueError("S must be a contiguous, 16-byte aligned float32 tensor (updated in place)")
    q, k, v, alpha, beta = map(_prep, (q, k, v, alpha, beta))
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    if S.shape != (N, H, d_v, d_k):
        raise ValueError("S must be [N, H, d_v, d_k]")
    if gc in _PER_CHANNEL and alpha.shape != q.shape:
        raise ValueError("per-channel alpha must be [N, H, d_k]")
    if gc in _PER_TOKEN and alpha.numel() != N * H:
        raise ValueError("scalar alpha must be [N, H]")
    if out is None:
        out = torch.empty((N, H, d_v), dtype=v.dtype, device=q.device)
    st = lib.kda_decode_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), gc, _ptr(beta), _ptr(S),
                                   N, H, d_k, d_v, float(scale) if scale else 0.0, dt, _ptr(out),
                                   _stream(q.device))
    if st != 0:
        raise KdaError("kda_decode_step_gated", st)
    return out


def decode_tokens(q, k, v, alpha, beta, S_in, S_out=None, scale=None, *, gate=None, out=None, act=0,
                  conv=None, conv_state=None, norm_weight=None, norm_eps=1e-6, out_gate=None):
    """Tk tokens per sequence in one launch: q, k [N, Tk, H, d_k]; v
    [N, Tk, H, d_v]; beta [N, Tk, H]; alpha [N, Tk, H, d_k] ("channel"),
    [N, Tk, H] ("scalar") or None ("none").  The state is read from S_in
    ([N, H, d_v, d_k] fp32) and the state after the last token is written to
    S_out: a new tensor by default, so S_in stays the checkpoint; pass
    S_out=S_in to update in place.  ``act`` as for chunk_fwd.  Module
    operations as for chunk_fwd (kda_decode_tokens_module): with ``conv``,
    ``conv_state`` [N, H, 3, 2 d_k + d_v] holds the three raw tokens before
    the first and is replaced by the last three.  Returns
    (o [N, Tk, H, d_v], S_out)."""
    import torch
    dt = _dtype_code(q)
    gc = _gate_code(gate, alpha, q)
    if gc == KDA_GATE_NONE:
        alpha = None
    if not S_in.is_contiguous() or S_in.dtype != torch.float32 or S_in.data_ptr() % 16:
        raise ValueError("S_in must be a contiguous, 16-byte aligned float32 tensor")
    q, k, v, alpha, beta = map(_prep, (q, k, v, alpha, beta))
    if q.dim() != 4:
        raise ValueError("q must be [N, Tk, H, d_k]")
    N, Tk, H, d_k = q.shape
    d_v = v.shape[-1]
    if k.shape != q.shape or v.shape != (N, Tk, H, d_v) or beta.numel() != N * Tk * H:
        raise ValueError("k, v, beta do not match q")
    if gc in _PER_CHANNEL and alpha.shape != q.shape:
        raise ValueError("per-channel alpha must be [N, Tk, H, d_k]")
    if gc in _PER_TOKEN and alpha.numel() != N * Tk * H:
        raise ValueError("scalar alpha must be [N, Tk, H]")
    if S_in.shape != (N, H, d_v, d_k):
        raise ValueError("S_in must be [N, H, d_v, d_k]")
    if S_out is None:
        S_out = torch.empty_like(S_in)
    elif (not S_out.is_contiguous() or S_out.dtype != torch.float32 or S_out.data_ptr() % 16
          or S_out.shape != S_in.shape):
        raise ValueError("S_out must be a contiguous, 16-byte aligned float32 tensor shaped like S_in")
    if out is None:
        out = torch.empty((N, Tk, H, d_v), dtype=v.dtype, device=q.device)
    if conv is not None or norm_weight is not None or out_gate is not None:
        ops, _keep = _module_ops(torch, H, d_k, d_v, v.dtype, N * Tk * H * d_v, conv, norm_weight, norm_eps,
                                 out_gate, conv_state, N * H)
        st = lib.kda_decode_tokens_module(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), gc, _ptr(beta), int(act),
                                          ctypes.byref(ops), _ptr(S_in), _ptr(S_out), N, Tk, H, d_k, d_v,
                                          float(scale) if scale else 0.0, dt, _ptr(out), _stream(q.device))
        if st != 0:
            raise KdaError("kda_decode_tokens_module", st)
        return out, S_out
    st = lib.kda_decode_tokens_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), gc, _ptr(beta), int(act),
                                  _ptr(S_in), _ptr(S_out), N, Tk, H, d_k, d_v, float(scale) if scale else 0.0,
                                  dt, _ptr(out), _stream(q.device))
    if st != 0:
        raise KdaError("kda_decode_tokens_ex", st)
    return out, S_out
