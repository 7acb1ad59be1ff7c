"""The C ABI library loads and exports what include/kda.h declares; host-side
argument validation returns the documented status codes (CPU only: every
call here is rejected before any HIP call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def kda():
    import linear_attention_kda_amd as pkg
    pkg.lib  # loads libkda.so (ImportError if it was not built)
    return pkg


def test_exports_every_declared_symbol(kda):
    declared = _declared_functions()
    assert declared == sorted(kda.EXPORTED)
    for name in declared:
        assert hasattr(kda.lib, name), f"{name} not exported"


def test_status_strings(kda):
    for s in range(14):
        assert kda.status_string(s) and kda.status_string(s) != "unknown status"
    assert kda.status_string(99) == "unknown status"


def test_workspace_size(kda):
    # dense: one record per (chunk, head); a record holds three 64 x d_k tiles,
    # two lower-triangular 64 x 64 tiles stored as the 1 KiB fragments of the
    # k-slabs that reach the diagonal (6 slabs of 32 columns in bf16) and d_k
    # floats, rounded up to 1 KiB
    rec = (3 * 64 * 128 * 2 + 2 * 6 * 1024 + 128 * 4 + 1023) // 1024 * 1024
    # after 64 control words (256 bytes: the status of the last call and the
    # overlapped schedule's counters), then one int32 ready flag per record,
    # rounded up to 256 bytes
    nrec = 4 * 32 * 16
    ready = (nrec * 4 + 255) // 256 * 256
    assert kda.chunk_fwd_workspace_size(4, 2048, 16, 128, 128, -1, kda.KDA_BF16) == 256 + nrec * rec + ready
    # no tokens: the control words alone
    assert kda.chunk_fwd_workspace_size(2, 0, 3, 32, 32, -1, kda.KDA_F32) == 256
    # packed: tables plus (ceil(T/64) + N) chunk slots
    packed = kda.chunk_fwd_workspace_size(1, 1000, 2, 64, 64, 5, kda.KDA_BF16)
    rec64 = (3 * 64 * 64 * 2 + 2 * 6 * 1024 + 64 * 4 + 1023) // 1024 * 1024
    assert packed >= (16 + 5) * 2 * rec64
    # few long heads: the split-sequence buffers follow (here 8 segments of 128
    # chunks: segment tables, 7 x 8 maps of (d_v + d_k) x d_k fp32, and the
    # start and end states of 8 x 8 segments)
    nrec = 1024 * 8
    base = 256 + nrec * rec + (nrec * 4 + 255) // 256 * 256
    split = 256 + 7 * 8 * 256 * 128 * 4 + 2 * 8 * 8 * 128 * 128 * 4
    assert kda.chunk_fwd_workspace_size(1, 65536, 8, 128, 128, -1, kda.KDA_BF16) == base + split
    # invalid sizes
    assert kda.chunk_fwd_workspace_size(1, 10, 2, 48, 64, -1, kda.KDA_BF16) == 0
    assert kda.chunk_fwd_workspace_size(1, 10, 0, 64, 64, -1, kda.KDA_BF16) == 0
    assert kda.chunk_fwd_workspace_size(1, 10, 2, 64, 64, -1, 7) == 0
    # 64 token rows of all heads' outputs must span less than 2^31 bytes in fp32
    assert kda.chunk_fwd_workspace_size(1, 10, 65536, 16, 128, -1, kda.KDA_BF16) == 0
    assert kda.chunk_fwd_workspace_size(1, 10, 65535, 16, 128, -1, kda.KDA_BF16) > 0
    assert kda.chunk_fwd_workspace_size(1, 10, 1 << 19, 16, 16, -1, kda.KDA_BF16) == 0


def _fwd(kda, **kw):
    """Call kda_chunk_fwd with fake (never dereferenced) aligned pointers."""
    P = lambda a: ctypes.c_void_p(a)
    args = dict(q=P(0x10000), k=P(0x20000), v=P(0x30000), alpha=P(0x40000), beta=P(0x50000),
                S0=None, cu=None, N=2, B=2, T=8, H=2, dk=16, dv=16, scale=0.0, dt=kda.KDA_BF16,
                o=P(0x60000), S_final=P(0x70000), ws=P(0x80000), ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return kda.lib.kda_chunk_fwd(args["q"], args["k"], args["v"], args["alpha"], args["beta"],
                                 args["S0"], args["cu"], args["N"], args["B"], args["T"], args["H"],
                                 args["dk"], args["dv"], args["scale"], args["dt"], args["o"],
                                 args["S_final"], args["ws"], args["ws_bytes"], args["stream"])


def test_chunk_fwd_validation(kda):
    P = ctypes.c_void_p
    assert _fwd(kda, dt=5) == 4                      # unsupported dtype
    assert _fwd(kda, dk=48) == 3                     # unsupported dim
    assert _fwd(kda, dv=256) == 3
    assert _fwd(kda, H=0) == 2                       # bad shape
    assert _fwd(kda, T=-1) == 2
    assert _fwd(kda, H=65536, dv=128) == 2           # H d_v >= 2^23
    assert _fwd(kda, H=1 << 19, dv=16) == 2
    assert _fwd(kda, H=65535, dv=128, S_final=None) == 1   # within the bound: the next check
    assert _fwd(kda, q=None) == 1                    # null input
    assert _fwd(kda, S_final=None) == 1
    assert _fwd(kda, o=P(0x60004)) == 5              # misaligned
    assert _fwd(kda, cu=P(0x90000), B=2) == 7        # packed needs B == 1
    assert _fwd(kda, ws_bytes=10) == 6               # workspace too small
    assert _fwd(kda, ws=None) == 6
    assert _fwd(kda, o=P(0x30000)) == 8              # o aliases v
    assert _fwd(kda, o=P(0x80000)) == 8              # o aliases the workspace
    assert _fwd(kda, S_final=P(0x10000)) == 8        # S_final aliases q
    assert _fwd(kda, S_final=P(0x80000)) == 8        # S_final aliases the workspace
    assert _fwd(kda, ws=P(0x30000)) == 8             # the workspace aliases v
    assert _fwd(kda, ws=P(0x50000)) == 8             # ... beta
    assert _fwd(kda, S0=P(0x70000 + 256)) == 8       # S0 overlaps S_final without being it
    assert _fwd(kda, S0=P(0x60000)) == 8             # S0 overlaps o
    assert _fwd(kda, S0=P(0x80000)) == 8             # S0 overlaps the workspace
    assert _fwd(kda, cu=P(0x70000), B=1) == 8        # the offsets overlap S_final


def test_decode_validation(kda):
    P = ctypes.c_void_p
    good = dict(q=P(0x10000), k=P(0x20000), v=P(0x30000), alpha=P(0x40000), beta=P(0x50000),
                S=P(0x60000), N=2, H=2, dk=16, dv=16, scale=0.0, dt=kda.KDA_F32, o=P(0x90000))

    def call(**kw):
        a = dict(good, **kw)
        return kda.lib.kda_decode_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S"], a["N"],
                                       a["H"], a["dk"], a["dv"], a["scale"], a["dt"], a["o"], None)
    assert call(dt=3) == 4
    assert call(dk=8) == 3
    assert call(H=0) == 2
    assert call(N=0) == 0                            # nothing to do
    assert call(S=None) == 1
    assert call(beta=P(0x50008)) == 5
    assert call(o=P(0x60000)) == 8                   # o aliases S
    assert call(S=P(0x10000)) == 8                   # the state overlaps q
    assert call(S=P(0x50000)) == 8                   # ... beta


def _fwd_gated(kda, gate, **kw):
    P = lambda a: ctypes.c_void_p(a)
    args = dict(q=P(0x10000), k=P(0x20000), v=P(0x30000), alpha=P(0x40000), beta=P(0x50000),
                S0=None, cu=None, N=2, B=2, T=8, H=2, dk=16, dv=16, scale=0.0, dt=kda.KDA_BF16,
                o=P(0x60000), S_final=P(0x70000), ws=P(0x80000), ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return kda.lib.kda_chunk_fwd_gated(args["q"], args["k"], args["v"], args["alpha"], gate, args["beta"],
                                       args["S0"], args["cu"], args["N"], args["B"], args["T"], args["H"],
                                       args["dk"], args["dv"], args["scale"], args["dt"], args["o"],
                                       args["S_final"], args["ws"], args["ws_bytes"], args["stream"])


def test_gated_validation(kda):
    P = ctypes.c_void_p
    assert _fwd_gated(kda, 7) == 10                           # unknown gate
    assert _fwd_gated(kda, 99) == 10
    assert _fwd_gated(kda, -1) == 10
    assert _fwd_gated(kda, kda.KDA_GATE_LOG_SCALAR, alpha=None) == 1   # log gates need alpha
    assert _fwd_gated(kda, kda.KDA_GATE_LOG_CHANNEL, alpha=P(0x40008)) == 5
    # a log per-channel gate has the per-channel extent: o inside it aliases
    assert _fwd_gated(kda, kda.KDA_GATE_LOG_CHANNEL, o=P(0x40000 + 256)) == 8
    assert _fwd_gated(kda, kda.KDA_GATE_SCALAR, alpha=None) == 1   # scalar gates need alpha
    assert _fwd_gated(kda, kda.KDA_GATE_CHANNEL, alpha=None) == 1
    assert _fwd_gated(kda, kda.KDA_GATE_SCALAR, alpha=P(0x40004)) == 5
    # no gate: alpha is not read, so NULL or a misaligned value are both fine;
    # the call then fails later on the deliberately bad shape
    assert _fwd_gated(kda, kda.KDA_GATE_NONE, alpha=None, H=0) == 2
    assert _fwd_gated(kda, kda.KDA_GATE_NONE, alpha=P(0x40004), dk=48) == 3
    # a scalar alpha covers B*T*H floats, a per-channel one B*T*H*d_k: o placed
    # inside the per-channel extent aliases only that form
    assert _fwd_gated(kda, kda.KDA_GATE_CHANNEL, o=P(0x40000 + 256)) == 8
    # decode
    good = dict(q=P(0x10000), k=P(0x20000), v=P(0x30000), beta=P(0x50000), S=P(0x60000), o=P(0x90000))

    def dec(gate, alpha, **kw):
        a = dict(good, **kw)
        return kda.lib.kda_decode_step_gated(a["q"], a["k"], a["v"], alpha, gate, a["beta"], a["S"], 2, 2,
                                             16, 16, 0.0, kda.KDA_F32, a["o"], None)
    assert dec(7, P(0x40000)) == 10
    assert dec(kda.KDA_GATE_LOG_CHANNEL, None) == 1
    assert dec(kda.KDA_GATE_LOG_SCALAR, P(0x40002)) == 5
    assert dec(kda.KDA_GATE_SCALAR, None) == 1
    assert dec(kda.KDA_GATE_CHANNEL, P(0x40008)) == 5
    assert dec(kda.KDA_GATE_NONE, None, o=P(0x60000)) == 8   # o aliases S, alpha unused


def test_decode_tokens_validation(kda):
    P = ctypes.c_void_p
    good = dict(q=P(0x10000), k=P(0x20000), v=P(0x30000), alpha=P(0x40000), beta=P(0x50000),
                Si=P(0x100000), So=P(0x200000), o=P(0x90000), N=2, Tk=3, H=2, gate=kda.KDA_GATE_CHANNEL)

    def call(**kw):
        a = dict(good, **kw)
        return kda.lib.kda_decode_tokens(a["q"], a["k"], a["v"], a["alpha"], a["gate"], a["beta"], a["Si"],
                                         a["So"], a["N"], a["Tk"], a["H"], 16, 16, 0.0, kda.KDA_F32, a["o"],
                                         None)
    assert call(Tk=-1) == 2
    assert call(gate=7) == 10
    assert call(Si=None) == 1
    assert call(So=P(0x100000 + 256)) == 8          # partial overlap of the two states
    assert call(o=P(0x100000)) == 8                 # o overlaps a state
    assert call(So=P(0x30000)) == 8                 # the output state overlaps v
    assert call(gate=kda.KDA_GATE_SCALAR, alpha=None) == 1
    assert call(N=0) == 0


def test_ex_rejects_unknown_activation_bits(kda):
    # rejected before any pointer is looked at or any work is launched
    P = ctypes.c_void_p
    st = kda.lib.kda_chunk_fwd_ex(P(0x10000), P(0x20000), P(0x30000), P(0x40000), kda.KDA_GATE_CHANNEL,
                                  P(0x50000), 4, None, None, 2, 2, 8, 2, 16, 16, 0.0, kda.KDA_BF16,
                                  P(0x60000), P(0x70000), P(0x80000), 1 << 30, None)
    assert st == 12
    st = kda.lib.kda_decode_tokens_ex(P(0x10000), P(0x20000), P(0x30000), P(0x40000), kda.KDA_GATE_CHANNEL,
                                      P(0x50000), 8, P(0x100000), P(0x200000), 2, 3, 2, 16, 16, 0.0,
                                      kda.KDA_F32, P(0x90000), None)
    assert st == 12
    assert kda.status_string(12) != "unknown status"


def test_set_validation_toggles(kda):
    # host-side switch only: no compute call is made here
    prev = kda.set_validation(True)
    try:
        assert kda.set_validation(True) is True
        assert kda.set_validation(False) is True
        assert kda.set_validation(False) is False
    finally:
        kda.set_validation(prev)


def test_status_query_and_release_host_checks(kda):
    # rejected before any device access
    P = ctypes.c_void_p
    sched, errs = ctypes.c_int(-7), ctypes.c_uint(7)
    assert kda.lib.kda_chunk_fwd_status(None, None, ctypes.byref(sched), ctypes.byref(errs)) == 1
    assert kda.lib.kda_chunk_fwd_status(P(0x80004), None, ctypes.byref(sched), ctypes.byref(errs)) == 5
    assert sched.value == -7 and errs.value == 7            # outputs untouched on error
    # nothing was created: release is a no-op, and may run any number of times
    kda.release()
    kda.release()


def test_set_validation_query(kda):
    prev = kda.set_validation(False)
    try:
        assert kda.lib.kda_set_validation(-1) == 0
        assert kda.validation_enabled() is False
        kda.set_validation(True)
        assert kda.lib.kda_set_validation(-1) == 1      # a query changes nothing
        assert kda.validation_enabled() is True
    finally:
        kda.set_validation(prev)


def _module(kda, ops, act=1, ws_bytes=10, **kw):
    """kda_chunk_fwd_module with fake aligned pointers; every case below is
    rejected on the host."""
    P = lambda a: ctypes.c_void_p(a)
    a = dict(q=P(0x10000), k=P(0x20000), v=P(0x30000), alpha=P(0x40000), beta=P(0x50000), o=P(0x60000),
             S_final=P(0x70000), ws=P(0x80000))
    a.update(kw)
    return kda.lib.kda_chunk_fwd_module(a["q"], a["k"], a["v"], a["alpha"], kda.KDA_GATE_CHANNEL, a["beta"], act,
                                        None if ops is None else ctypes.byref(ops), None, None, 2, 2, 8, 2, 16,
                                        16, 0.0, kda.KDA_BF16, a["o"], a["S_final"], a["ws"], ws_bytes, None)


def test_module_ops_host_checks(kda):
    from linear_attention_kda_amd._binding import KdaModuleOps
    W = [0x100000, 0x101000, 0x102000]
    # ops == NULL is kda_chunk_fwd_ex: the workspace of 10 bytes is too small
    assert _module(kda, None) == 6
    # only some of the convolution weights
    assert _module(kda, KdaModuleOps(W[0], W[1], None, None, 0.0, None)) == 1
    assert _module(kda, KdaModuleOps(None, None, W[2], None, 0.0, None)) == 1
    # the convolution needs the q, k activation
    assert _module(kda, KdaModuleOps(W[0], W[1], W[2], None, 0.0, None), act=0) == 12
    assert _module(kda, KdaModuleOps(W[0], W[1], W[2], None, 0.0, None), act=2) == 12
    # negative or NaN eps with a norm
    assert _module(kda, KdaModuleOps(None, None, None, 0x103000, -1.0, None)) == 2
    assert _module(kda, KdaModuleOps(None, None, None, 0x103000, float("nan"), None)) == 2
    # misaligned weight or gate
    assert _module(kda, KdaModuleOps(W[0] + 4, W[1], W[2], None, 0.0, None)) == 5
    assert _module(kda, KdaModuleOps(None, None, None, None, 0.0, 0x104008)) == 5
    # o overlapping a weight or the gate (checked after the workspace size)
    big = 1 << 30
    assert _module(kda, KdaModuleOps(W[0], W[1], W[2], None, 0.0, None), ws_bytes=big, o=ctypes.c_void_p(W[1])) == 8
    assert _module(kda, KdaModuleOps(None, None, None, 0x103000, 1e-6, None), ws_bytes=big,
                   o=ctypes.c_void_p(0x103000)) == 8
    assert _module(kda, KdaModuleOps(None, None, None, None, 0.0, 0x60000 + 512), ws_bytes=big) == 8
    # valid ops, then the workspace check as for kda_chunk_fwd_ex
    assert _module(kda, KdaModuleOps(W[0], W[1], W[2], 0x103000, 1e-6, 0x104000)) == 6
