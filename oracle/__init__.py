"""fp64 CPU oracle of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library does not depend on it
and it does not depend on the GPU library: the two share no code.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, token by token; see
its header for the recurrence and the citations).  This module only builds it
with gcc, widens inputs exactly to float64 and marshals arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def compile_source(src: str, lib: str) -> str:
    """gcc the oracle source ``src`` into the shared library ``lib``
    (no fast-math, no FP contraction)."""
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                           "-shared", "-fPIC", "-pthread", src, "-o", tmp, "-lm"])
    os.replace(tmp, lib)
    return lib


def build(force: bool = True) -> str:
    """Compile the oracle library next to its source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def open_library(path: str):
    """ctypes handle of an oracle library at ``path``, with signatures set."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.gdn_oracle_prefill.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, I, I]
    lib.gdn_oracle_prefill.restype = I
    lib.gdn_oracle_decode.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I]
    lib.gdn_oracle_decode.restype = I
    L = ctypes.c_long
    lib.gdn_oracle_ba_gates.argtypes = [P, P, P, P, P, I, I, I, L, L, I, I]
    lib.gdn_oracle_ba_gates.restype = I
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = open_library(_LIB)
    return _lib


def _f64(x):
    """Exact widening to a C-contiguous float64 array (accepts numpy or torch)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (any float dtype): widen in torch, exactly
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def prefill(q, k, v, log_g, beta, h0=None, cu_seqlens=None, heads=None, nthreads=None,
            want_out=True, want_state=True, lib=None):
    """Token-by-token fp64 gated delta rule over B sequences.

    Dense: q, k [B, T, Hk, dk]; v [B, T, Hv, dv]; log_g, beta [B, T, Hv].
    Packed: q, k [N, Hk, dk]; v [N, Hv, dv]; log_g, beta [N, Hv] with
    cu_seqlens [B+1].  h0: [B, Hv, dk, dv] or None (zeros).
    heads: optional iterable of v-heads to compute (others stay NaN).
    Returns (out with v's row shape, h_final [B, Hv, dk, dv]).
    """
    q, k, v, log_g, beta, h0 = (_f64(a) for a in (q, k, v, log_g, beta, h0))
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        B = cu.size - 1
        N, Hk, dk = q.shape
        T = 0
        assert cu[-1] == N
    else:
        cu = None
        B, T, Hk, dk = q.shape
    Hv, dv = v.shape[-2], v.shape[-1]
    hl = None
    if heads is not None:
        hl = np.ascontiguousarray(np.asarray(list(heads), dtype=np.int32))
    out = np.full(v.shape, np.nan) if want_out else None
    hf = np.full((B, Hv, dk, dv), np.nan) if want_state else None
    rc = (lib or _load()).gdn_oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta), _ptr(h0),
                                    _ptr(out), _ptr(hf), B, T, Hk, Hv, dk, dv, _ptr(cu), _ptr(hl),
                                    0 if hl is None else hl.size,
                                    nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle prefill: bad shape")
    return out, hf


def decode(states, q, k, v, gate, beta, lib=None):
    """K draft rows per sequence from per-sequence states.

    states [B, Hv, dk, dv]; q, k [B, K, Hk, dk]; v [B, K, Hv, dv];
    gate, beta [B, K, Hv].  Returns (out [B, K, Hv, dv],
    after [B, K+1, Hv, dk, dv]) where after[:, r] is the state once the
    first r rows are applied (after[:, 0] is the input state).
    """
    states, q, k, v, gate, beta = (_f64(a) for a in (states, q, k, v, gate, beta))
    B, K, Hk, dk = q.shape
    Hv, dv = v.shape[-2], v.shape[-1]
    out = np.zeros((B, K, Hv, dv))
    after = np.zeros((B, K + 1, Hv, dk, dv))
    rc = (lib or _load()).gdn_oracle_decode(_ptr(states), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                                   _ptr(out), _ptr(after), B, K, Hk, Hv, dk, dv)
    if rc != 0:
        raise ValueError("oracle decode: bad shape")
    return out, after


def ba_gates(x, w, a_log, dt_bias, nv, vheads_per_group, lib=None):
    """The gate/beta producer: x [m, k] (or [m, x_stride] with the first k
    columns used, k = w.shape[1]), w [2 nv, k], a_log and dt_bias [nv].
    Returns out [m, 2 nv]: columns 0..nv-1 the log-decay gate, nv..2nv-1 beta.
    """
    x, w, a_log, dt_bias = (_f64(a) for a in (x, w, a_log, dt_bias))
    m, x_stride = x.shape
    n, k = w.shape
    out = np.full((m, 2 * nv), np.nan)
    rc = (lib or _load()).gdn_oracle_ba_gates(_ptr(x), _ptr(w), _ptr(a_log), _ptr(dt_bias), _ptr(out),
                                              m, n, k, x_stride, 2 * nv, nv, vheads_per_group)
    if rc != 0:
        raise ValueError("oracle ba_gates: bad shape")
    return out
