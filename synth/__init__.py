"""Seeded synthetic inputs for the gated delta rule.

This module draws and rounds inputs; it holds none of the method's arithmetic.
Both the fp64 oracle and the GPU library are fed from here, so that parity
tests compare the two on identical bytes.

Recipe (per workload below):
  * q, k ~ N(0, 1) in fp64, L2-normalised per (token, head) in fp64, then
    rounded to fp32 (RNE) and, for bf16 workloads, to bf16 (RNE);
  * v ~ N(0, 1), rounded the same way;
  * log_g = -softplus(x) * 0.1 with x ~ N(0, 1), softplus(x) = log(1 + e^x),
    rounded to fp32;  beta = sigmoid(y) with y ~ N(0, 1), rounded to fp32;
  * h0: zeros (passed as "no initial state") or N(0, 0.02^2) (0.02 is the
    standard deviation) in fp32, one dk x dv state per (sequence, v-head);
  * packed sequences: lengths uniform on the integers of [lo, hi].
The gate/beta producer (BA projection) takes, in place of a model's trained
weights and activations:
  * activations x ~ N(0, 1), rounded to bf16;
  * the weight [2 nv][k] ~ N(0, 1/k) (unit-variance pre-activations), bf16;
  * a_log = ln(A) with A ~ U(1, 16), and dt_bias = ln(e^dt - 1) with
    ln(dt) ~ U(ln 0.001, ln 0.1), both fp32 (the usual initialisation of
    these two parameters in Mamba-style gating).
The generator is numpy's PCG64 (``numpy.random.default_rng(seed)``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


def _round(x64: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """fp64 -> fp32 (RNE) -> dtype (RNE when dtype is bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _gates(rng: np.random.Generator, shape, scale=0.1):
    x = rng.standard_normal(shape)
    log_g = -np.logaddexp(0.0, x) * scale        # -softplus(x) * scale
    y = rng.standard_normal(shape)
    beta = 1.0 / (1.0 + np.exp(-y))              # sigmoid(y)
    return log_g, beta


@dataclass(frozen=True)
class Workload:
    """A named prefill or decode workload."""
    name: str
    kind: str                  # "prefill" or "decode"
    B: int
    T: int                     # tokens per sequence (dense) or 0 when packed
    Hk: int
    Hv: int
    dk: int
    dv: int
    chunk: int = 64
    io: torch.dtype = torch.bfloat16
    h0: bool = False
    seed: int = 0
    packed: Optional[tuple] = None   # (lo, hi) sequence-length range when packed
    k_rows: int = 4                  # decode rows per sequence
    note: str = ""


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32", "prefill", B=1, T=128, Hk=1, Hv=1, dk=32, dv=32, chunk=32,
                 io=torch.float32, h0=False, seed=1000,
                 note="fp32 gated delta rule, one head, d=32, chunk 32"),
        Workload("prefill_t1168", "prefill", B=1, T=1168, Hk=16, Hv=48, dk=128, dv=128, chunk=64,
                 io=torch.bfloat16, h0=False, seed=1001,
                 note="one 1168-token prefill call, 48 v-heads over 16 k-heads, no initial state"),
        Workload("prefill_t4576_h0", "prefill", B=1, T=4576, Hk=16, Hv=48, dk=128, dv=128, chunk=64,
                 io=torch.bfloat16, h0=True, seed=1002,
                 note="one 4576-token prefill call with an initial state"),
        Workload("prefill_t4576_hv6", "prefill", B=1, T=4576, Hk=2, Hv=6, dk=128, dv=128, chunk=64,
                 io=torch.bfloat16, h0=True, seed=1007,
                 note="one 4576-token prefill call of a narrow layer: 6 v-heads over 2 k-heads"),
        Workload("varlen_b8", "prefill", B=8, T=0, Hk=16, Hv=48, dk=128, dv=128, chunk=64,
                 io=torch.bfloat16, h0=True, seed=1003, packed=(1600, 8192),
                 note="8 packed sequences of 1600..8192 tokens, per-sequence states"),
        Workload("verify_k4_b16", "decode", B=16, T=4, Hk=16, Hv=48, dk=128, dv=128,
                 io=torch.bfloat16, h0=True, seed=1004, k_rows=4,
                 note="K=4 draft verify of 16 sequences, states behind a pointer table"),
        Workload("step_b16", "decode_step", B=16, T=1, Hk=16, Hv=48, dk=128, dv=128,
                 io=torch.bfloat16, h0=True, seed=1005, k_rows=1,
                 note="single-token decode step of 16 sequences, states updated in place"),
    ]
}


# The gate/beta producer at the pages' geometry: one 4576-token prefill's
# activations (hidden size 5120) against 2 x 48 BA outputs, 3 v-heads per
# k-head group.
BA_WORKLOAD = dict(name="ba_gates_t4576", m=4576, k=5120, nv=48, vheads_per_group=3, seed=1006)


def ba_inputs(m, k, nv, seed=0, x_stride=None):
    """Inputs of one gate/beta producer call as CPU tensors: x bf16
    [m, x_stride] (columns k.. are filled too, and must be ignored), w bf16
    [2 nv, k], a_log and dt_bias fp32 [nv]."""
    rng = np.random.default_rng(seed)
    xs = k if x_stride is None else x_stride
    x = _round(rng.standard_normal((m, xs)), torch.bfloat16)
    w = _round(rng.standard_normal((2 * nv, k)) / np.sqrt(k), torch.bfloat16)
    a_log = _round(np.log(rng.uniform(1.0, 16.0, nv)), torch.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), nv))
    dt_bias = _round(np.log(np.expm1(dt)), torch.float32)
    return dict(x=x, w=w, a_log=a_log, dt_bias=dt_bias)


def packed_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=B)


def prefill_inputs(B, T, Hk, Hv, dk, dv, io=torch.bfloat16, h0=False, seed=0, lengths=None,
                   gate_scale=0.1):
    """Inputs of one prefill call as CPU tensors (log_g = -gate_scale
    softplus(x), x standard normal: a mean decay of about 0.08 per token at
    the default, so a state forgets most of itself within ~50 tokens).

    Dense (lengths is None): q, k [B, T, Hk, dk]; v [B, T, Hv, dv];
    log_g, beta [B, T, Hv].  Packed (lengths given): rows of all sequences
    concatenated: q, k [N, Hk, dk] ... with cu_seqlens int32 [B+1].
    """
    rng = np.random.default_rng(seed)
    if lengths is None:
        rows = (B, T)
        cu = None
    else:
        lengths = np.asarray(lengths, dtype=np.int64)
        assert lengths.size == B
        rows = (int(lengths.sum()),)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    q = _unit_rows(rng, rows + (Hk, dk))
    k = _unit_rows(rng, rows + (Hk, dk))
    v = rng.standard_normal(rows + (Hv, dv))
    log_g, beta = _gates(rng, rows + (Hv,), gate_scale)
    d = dict(q=_round(q, io), k=_round(k, io), v=_round(v, io),
             log_g=_round(log_g, torch.float32), beta=_round(beta, torch.float32),
             h0=None, cu_seqlens=cu)
    if h0:
        d["h0"] = _round(rng.standard_normal((B, Hv, dk, dv)) * 0.02, torch.float32)
    return d


def workload_inputs(w: Workload):
    """Inputs of a named prefill workload (see WORKLOADS)."""
    assert w.kind == "prefill"
    lengths = None
    if w.packed is not None:
        lengths = packed_lengths(w.B, w.packed[0], w.packed[1], w.seed + 1)
    return prefill_inputs(w.B, w.T, w.Hk, w.Hv, w.dk, w.dv, io=w.io, h0=w.h0, seed=w.seed,
                          lengths=lengths)


def decode_inputs(B, K, Hk, Hv, dk, dv, io=torch.bfloat16, seed=0):
    """Inputs of one K-row verify: per-sequence states, K rows per sequence,
    and accept counts na in {0..K} (the first K+1 sequences take 0..K, so
    every count occurs; the rest are uniform)."""
    rng = np.random.default_rng(seed)
    states = rng.standard_normal((B, Hv, dk, dv)) * 0.02
    q = _unit_rows(rng, (B, K, Hk, dk))
    k = _unit_rows(rng, (B, K, Hk, dk))
    v = rng.standard_normal((B, K, Hv, dv))
    gate, beta = _gates(rng, (B, K, Hv))
    na = rng.integers(0, K + 1, size=B)
    na[: min(B, K + 1)] = np.arange(min(B, K + 1))
    return dict(states=_round(states, torch.float32), q=_round(q, io), k=_round(k, io),
                v=_round(v, io), gate=_round(gate, torch.float32),
                beta=_round(beta, torch.float32),
                na=torch.from_numpy(na.astype(np.int32)),
                slot_perm=torch.from_numpy(rng.permutation(B).astype(np.int64)))


def max_rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor, in fp64."""
    g = got.detach().to("cpu", torch.float64).numpy() if hasattr(got, "detach") else np.asarray(got, np.float64)
    r = ref.detach().to("cpu", torch.float64).numpy() if hasattr(ref, "detach") else np.asarray(ref, np.float64)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / (den if den > 0 else 1.0))
