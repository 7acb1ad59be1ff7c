"""fp64 CPU oracle of the KDA recurrence -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, token by token); it
follows page "Kimi Delta Attention (KDA)" (brain.bigb.es), opening update
equation and section "KDA: a separate gate per key channel".  This module
only builds that file with gcc and marshals arrays through ctypes: every
input is upcast exactly to float64 (bf16 and fp32 values are representable),
and outputs come back as float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import shlex
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kda_oracle.c")
# KDA_ORACLE_LIB and KDA_ORACLE_CFLAGS let a test job build and load the
# oracle elsewhere and with extra compiler flags (the sanitizer job does)
LIB_PATH = os.environ.get("KDA_ORACLE_LIB") or os.path.join(_HERE, "libkda_oracle.so")

_DP = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)


def compile_oracle(source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle C source into a shared library with gcc."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           *shlex.split(os.environ.get("KDA_ORACLE_CFLAGS", "")), "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _to_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or CPU/GPU torch tensor to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(_DP)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, lib_path: str = LIB_PATH):
        if not os.path.exists(lib_path):
            compile_oracle(out=lib_path)
        self.lib = ctypes.CDLL(lib_path)
        self.lib.kda_oracle_fwd.restype = ctypes.c_int
        self.lib.kda_oracle_fwd.argtypes = [
            _DP, _DP, _DP, _DP, _DP, _DP, _I64P, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, _DP,
            _DP, ctypes.c_int]
        self.lib.kda_oracle_decode.restype = ctypes.c_int
        self.lib.kda_oracle_decode.argtypes = [
            _DP, _DP, _DP, _DP, _DP, _DP, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, _DP, ctypes.c_int]

    def fwd(self, q, k, v, alpha, beta, S0=None, cu_seqlens=None, scale=None,
            n_threads=None):
        """Forward over whole sequences.

        Dense batch: q,k,alpha [B,T,H,dk], v [B,T,H,dv], beta [B,T,H].
        Packed batch (cu_seqlens given, length N+1): leading dim is the packed
        token axis, i.e. [Ttot,H,dk] (a leading batch dim of 1 is accepted).
        S0: [N,H,dv,dk] or None.  Returns (o, S_final) as float64 arrays with
        o shaped like v.
        """
        q, k, v, alpha, beta = map(_to_f64, (q, k, v, alpha, beta))
        out_shape = v.shape
        dk, dv = q.shape[-1], v.shape[-1]
        H = q.shape[-2]
        if cu_seqlens is not None:
            cu = np.ascontiguousarray(np.asarray(
                cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                dtype=np.int64))
            N = cu.shape[0] - 1
            T = 0
            ttot = int(cu[-1])
        else:
            cu = None
            N, T = q.shape[0], q.shape[1]
            ttot = N * T
        for name, a, last in (("q", q, dk), ("k", k, dk), ("alpha", alpha, dk),
                              ("v", v, dv)):
            if a.size != ttot * H * last:
                raise ValueError(f"{name} has {a.size} elements, expected "
                                 f"{ttot * H * last}")
        if beta.size != ttot * H:
            raise ValueError("beta size mismatch")
        S0 = _to_f64(S0)
        if S0 is not None and S0.size != N * H * dv * dk:
            raise ValueError("S0 size mismatch")
        o = np.zeros(out_shape, dtype=np.float64)
        S_final = np.zeros((N, H, dv, dk), dtype=np.float64)
        rc = self.lib.kda_oracle_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0),
            cu.ctypes.data_as(_I64P) if cu is not None else None, N, T, H, dk,
            dv, float(scale) if scale else 0.0, _ptr(o), _ptr(S_final),
            int(n_threads or default_threads()))
        if rc != 0:
            raise ValueError(f"kda_oracle_fwd returned {rc}")
        return o, S_final

    def decode(self, q, k, v, alpha, beta, S, scale=None, n_threads=None):
        """One token for each of N sequences.  q,k,alpha [N,H,dk], v [N,H,dv],
        beta [N,H]; S [N,H,dv,dk].  Returns (o, S_new) as float64 arrays; the
        caller's S is not modified."""
        q, k, v, alpha, beta = map(_to_f64, (q, k, v, alpha, beta))
        S_new = _to_f64(S).copy()
        N, H, dk = q.shape
        dv = v.shape[-1]
        o = np.zeros((N, H, dv), dtype=np.float64)
        rc = self.lib.kda_oracle_decode(
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S_new),
            N, H, dk, dv, float(scale) if scale else 0.0, _ptr(o),
            int(n_threads or default_threads()))
        if rc != 0:
            raise ValueError(f"kda_oracle_decode returned {rc}")
        return o, S_new


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``kda_oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def fwd(*args, **kwargs):
    return get().fwd(*args, **kwargs)


def decode(*args, **kwargs):
    return get().decode(*args, **kwargs)


def rel_l2(x, ref) -> float:
    """Relative L2 error ||x - ref|| / ||ref|| over the whole array, in fp64."""
    x = _to_f64(x)
    ref = _to_f64(ref)
    num = float(np.linalg.norm((x - ref).ravel()))
    den = float(np.linalg.norm(ref.ravel()))
    if den == 0.0:
        return num
    return num / den


def unit_rel_l2(x, ref, unit_axes=(0, 1), cu_seqlens=None) -> np.ndarray:
    """Relative L2 error of every (sequence, head) unit, in fp64.

    Dense layout: ``unit_axes`` names the sequence axis and the head axis;
    the error and the reference norm are summed over every other axis.
    Packed layout (``cu_seqlens`` given, length N+1): axis 0 is the packed
    token axis and axis 1 the head axis; sequence n owns tokens
    [cu[n], cu[n+1]).  Returns an array [sequences, heads]; a unit whose
    reference is all zero reports its absolute error, as rel_l2 does."""
    x = _to_f64(x)
    ref = _to_f64(ref)
    if x.shape != ref.shape:
        raise ValueError(f"shapes differ: {x.shape} vs {ref.shape}")
    d2 = (x - ref) ** 2
    r2 = ref ** 2
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                        dtype=np.int64)
        rest = tuple(range(2, x.ndim))
        d2t, r2t = d2.sum(axis=rest), r2.sum(axis=rest)      # [tokens, heads]
        N = cu.shape[0] - 1
        num = np.zeros((N, x.shape[1]))
        den = np.zeros((N, x.shape[1]))
        for n in range(N):
            a, b = int(cu[n]), int(cu[n + 1])
            num[n] = d2t[a:b].sum(axis=0)
            den[n] = r2t[a:b].sum(axis=0)
    else:
        a0, a1 = unit_axes
        rest = tuple(i for i in range(x.ndim) if i not in (a0, a1))
        num = d2.sum(axis=rest)
        den = r2.sum(axis=rest)
        if a0 > a1:
            num, den = num.T, den.T
    num, den = np.sqrt(num), np.sqrt(den)
    return np.where(den > 0.0, num / np.where(den > 0.0, den, 1.0), num)
