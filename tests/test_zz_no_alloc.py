"""GPU check of gdn_chunk_prefill_noalloc (the entry point for callers that
cannot allocate): called through the C ABI twice in a row, the second call
smaller than the first, each output and final state must equal, bit for bit,
what gdn_chunk_prefill with a torch-allocated workspace returns for the same
inputs (same kernels, same arithmetic); the small call is also checked against
the fp64 oracle at the bf16 tolerance.
"""
import pytest
import torch

import linear_attention_ssm_gated_amd as gdn
import synth
from gpu_common import dev, oracle_prefill, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def _shapes(inp):
    cu = inp["cu_seqlens"]
    if cu is not None:
        B = cu.numel() - 1
        T, Hk, dk = inp["q"].shape
    else:
        B, T, Hk, dk = inp["q"].shape
    Hv, dv = inp["v"].shape[-2], inp["v"].shape[-1]
    return B, T, Hk, Hv, dk, dv


def _run_both(inp):
    g = to_dev(inp)
    B, T, Hk, Hv, dk, dv = _shapes(inp)
    ws_n = gdn.gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, 64, gdn.GDN_BF16,
                                           packed=g["cu_seqlens"] is not None)
    assert 0 < ws_n <= gdn.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev())
    ref_o = torch.empty(g["v"].shape, dtype=torch.bfloat16, device=dev())
    ref_h = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev())
    gdn.gdn_chunk_prefill(g["q"], g["k"], g["v"], g["log_g"], g["beta"], g["h0"], ref_o, ref_h,
                          B, T, Hk, Hv, dk, dv, 64, cu_seqlens=g["cu_seqlens"], workspace=ws)
    out = torch.full_like(ref_o, float("nan"))
    hf = torch.full_like(ref_h, float("nan"))
    route = gdn.gdn_chunk_prefill_noalloc(g["q"], g["k"], g["v"], g["log_g"], g["beta"], g["h0"],
                                          out, hf, B, T, Hk, Hv, dk, dv, 64,
                                          cu_seqlens=g["cu_seqlens"])
    torch.cuda.synchronize()
    return out, hf, ref_o, ref_h, route


def test_noalloc_equals_workspace_entry_on_two_calls():
    big = synth.workload_inputs(synth.WORKLOADS["prefill_t4576_h0"])
    say("noalloc call 1: prefill_t4576_h0")
    o1, h1, r1, rh1, route = _run_both(big)
    assert route.startswith("gdn_wy_prep_kernel"), route
    assert torch.equal(o1, r1) and torch.equal(h1, rh1)

    small = synth.prefill_inputs(3, 0, 2, 6, 128, 128, h0=True, seed=77, lengths=[130, 1, 64])
    say("noalloc call 2: packed 130+1+64 tokens, Hv=6")
    o2, h2, r2, rh2, _ = _run_both(small)
    assert torch.equal(o2, r2) and torch.equal(h2, rh2)
    ro, rh = oracle_prefill(small)
    assert rel_err(o2, ro) <= 2e-2
    assert rel_err(h2, rh, head_axis=1) <= 2e-2
