"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import linear_attention_ssm_gated_amd as gdn
import oracle
import synth


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch.device("cuda:0")


def say(*a):
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(d):
    return {k: (v.to(dev()) if torch.is_tensor(v) else v) for k, v in d.items()}


def gpu_prefill(inp, chunk, out_dtype=None, want_state=True, h0=None, segmented=False):
    g = to_dev(inp)
    h0 = g["h0"] if h0 is None else h0
    out, hf, route = gdn.chunk_prefill(g["q"], g["k"], g["v"], g["log_g"], g["beta"], h0,
                                       cu_seqlens=g["cu_seqlens"], chunk=chunk,
                                       out_dtype=out_dtype, want_state=want_state,
                                       segmented=segmented)
    torch.cuda.synchronize()
    return out, hf, route


def oracle_prefill(inp, heads=None):
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy()
    return oracle.prefill(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["beta"], inp["h0"],
                          cu_seqlens=cu, heads=heads)


def rel_err(got, ref, heads=None, head_axis=-2):
    """max|got - ref| / max|ref| in fp64 over the whole tensor (or the listed v-heads)."""
    g = got.detach().to("cpu", torch.float64).numpy()
    r = np.asarray(ref, dtype=np.float64)
    if heads is not None:
        g = np.take(g, heads, axis=head_axis)
        r = np.take(r, heads, axis=head_axis)
    return synth.max_rel_err(g, r)
