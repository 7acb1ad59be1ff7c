"""Valid calls through the whole host path of the C ABI (argument checks,
alias checks, workspace planning, argument packing), run only against the
host-only build of kda_api.cpp with the stand-ins of host_stubs.cpp, under
the address and undefined-behaviour sanitizers (tests/test_sanitizers.py
starts it).  Pointers are fake but aligned and disjoint: nothing touches a
device.  Not collected by the normal test run (no test_ prefix)."""
import ctypes
import os

import pytest

import linear_attention_kda_amd as kda

P = ctypes.c_void_p
GB = 1 << 30


@pytest.fixture(autouse=True)
def stub_lib():
    if not hasattr(kda.lib, "kda_stub_calls"):
        pytest.skip("needs the host-only stub build (KDA_LIBRARY)")
    kda.lib.kda_stub_calls.restype = ctypes.c_int
    kda.lib.kda_stub_calls.argtypes = [ctypes.c_int]
    kda.lib.kda_stub_calls(-1)
    yield
    assert kda.lib.kda_stub_calls(3) == 0, "a launcher received an inconsistent plan"


def _ptrs():
    # one region of 4 GiB per argument, far apart: no two overlap
    base = 1 << 40
    return {name: base + i * (4 * GB) for i, name in enumerate(
        ("q", "k", "v", "alpha", "beta", "S0", "cu", "o", "S", "ws"))}


@pytest.mark.parametrize("B,T,H,dk,dv,dt", [(4, 2048, 16, 128, 128, 1), (1, 65536, 32, 128, 128, 1),
                                            (2, 1, 3, 16, 64, 0), (3, 130, 2, 64, 32, 0), (2, 0, 2, 32, 32, 1)])
@pytest.mark.parametrize("gate", [0, 1, 2, 3, 4, 5, 6])
def test_dense_calls(B, T, H, dk, dv, dt, gate):
    p = _ptrs()
    need = kda.lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, -1, dt)
    assert need >= 256
    for s0 in (None, p["S0"], p["S"]):          # no S0, S0, in place
        st = kda.lib.kda_chunk_fwd_ex(P(p["q"]), P(p["k"]), P(p["v"]), P(p["alpha"]), gate, P(p["beta"]),
                                      3, P(s0) if s0 else None, None, B, B, T, H, dk, dv, 0.0, dt, P(p["o"]),
                                      P(p["S"]), P(p["ws"]), need, None)
        assert st == 0
    assert kda.lib.kda_stub_calls(0) == 3
    # one byte short of the plan is refused before any launch
    st = kda.lib.kda_chunk_fwd(P(p["q"]), P(p["k"]), P(p["v"]), P(p["alpha"]), P(p["beta"]), None, None, B, B, T,
                               H, dk, dv, 0.0, dt, P(p["o"]), P(p["S"]), P(p["ws"]), need - 1, None)
    assert st == 6 and kda.lib.kda_stub_calls(0) == 3


@pytest.mark.parametrize("N,T", [(64, 274_797), (5, 1000), (1, 0), (0, 0), (3, 7)])
def test_packed_calls(N, T):
    p = _ptrs()
    need = kda.lib.kda_chunk_fwd_workspace_size(1, T, 16, 128, 128, N, 1)
    st = kda.lib.kda_chunk_fwd(P(p["q"]), P(p["k"]), P(p["v"]), P(p["alpha"]), P(p["beta"]), P(p["S0"]),
                               P(p["cu"]), N, 1, T, 16, 128, 128, 0.0, 1, P(p["o"]), P(p["S"]), P(p["ws"]), need,
                               None)
    assert st == 0
    assert kda.lib.kda_stub_calls(0) == (1 if N > 0 else 0)


def test_validation_path_runs_the_check_once_per_call():
    p = _ptrs()
    prev = kda.set_validation(True)
    try:
        need = kda.lib.kda_chunk_fwd_workspace_size(2, 100, 2, 32, 32, -1, 0)
        st = kda.lib.kda_chunk_fwd(P(p["q"]), P(p["k"]), P(p["v"]), P(p["alpha"]), P(p["beta"]), None, None, 2,
                                   2, 100, 2, 32, 32, 0.0, 0, P(p["o"]), P(p["S"]), P(p["ws"]), need, None)
        assert st == 0 and kda.lib.kda_stub_calls(2) == 1
    finally:
        kda.set_validation(prev)


@pytest.mark.parametrize("Tk,inplace", [(0, True), (1, True), (4, False), (7, True)])
def test_decode_calls(Tk, inplace):
    p = _ptrs()
    st = kda.lib.kda_decode_step(P(p["q"]), P(p["k"]), P(p["v"]), P(p["alpha"]), P(p["beta"]), P(p["S"]), 256,
                                 32, 128, 128, 0.0, 1, P(p["o"]), None)
    assert st == 0
    assert kda.lib.kda_stub_calls(4) == 0, "the plain step passed module operations to the launcher"
    S_out = p["S"] if inplace else p["S0"]
    st = kda.lib.kda_decode_tokens_ex(P(p["q"]), P(p["k"]), P(p["v"]), P(p["alpha"]), 0, P(p["beta"]), 3,
                                      P(p["S"]), P(S_out), 256, Tk, 32, 128, 128, 0.0, 1, P(p["o"]), None)
    assert st == 0
    assert kda.lib.kda_stub_calls(4) == 0
    assert kda.lib.kda_stub_calls(1) == 2


def test_status_query_reads_the_words():
    sched, errs = ctypes.c_int(-1), ctypes.c_uint(9)
    st = kda.lib.kda_chunk_fwd_status(P(_ptrs()["ws"]), None, ctypes.byref(sched), ctypes.byref(errs))
    assert st == 0 and sched.value == 0 and errs.value == 0
    kda.release()


def test_environment_is_the_stub_build():
    assert os.environ.get("KDA_LIBRARY", "").endswith("libkda_host_san.so")


@pytest.mark.parametrize("B,T,H,segments", [(4, 2048, 16, 4), (2, 8192, 64, 16), (1, 300, 4, 1), (2, 0, 3, 1)])
def test_noalloc_segments(B, T, H, segments):
    """The no-allocation entry point: a batch that fits runs as one launch,
    a larger one as segments of whole chunks per sequence (64 MiB scratch:
    16 heads x 32 chunks of 61 KiB fit, 64 heads fit 16 chunks)."""
    p = _ptrs()
    st = kda.lib.kda_chunk_fwd_noalloc(P(p["q"]), P(p["k"]), P(p["v"]), P(p["alpha"]), 0, P(p["beta"]), 0,
                                       P(p["S0"]), None, B, B, T, H, 128, 128, 0.0, 1, P(p["o"]), P(p["S"]), None)
    assert st == 0
    assert kda.lib.kda_stub_calls(0) == segments


def test_noalloc_limits():
    p = _ptrs()
    # one chunk of 1100 heads does not fit
    st = kda.lib.kda_chunk_fwd_noalloc(P(p["q"]), P(p["k"]), P(p["v"]), P(p["alpha"]), 0, P(p["beta"]), 0, None,
                                       None, 1, 1, 64, 1100, 128, 128, 0.0, 1, P(p["o"]), P(p["S"]), None)
    assert st == 14 and kda.lib.kda_stub_calls(0) == 0
    # a packed batch must fit whole
    st = kda.lib.kda_chunk_fwd_noalloc(P(p["q"]), P(p["k"]), P(p["v"]), P(p["alpha"]), 0, P(p["beta"]), 0, None,
                                       P(p["cu"]), 1, 1, 70_000, 16, 128, 128, 0.0, 1, P(p["o"]), P(p["S"]), None)
    assert st == 14 and kda.lib.kda_stub_calls(0) == 0
