"""GPU parity of the generic (fp32-arithmetic) chunked prefill against the fp64
oracle: max|d|/max|ref| <= 1e-4 on outputs and final states (fp32 outputs).

Covers the tiny fp32 workload (B=1, T=128, one head, d=32, chunk 32) and
shapes that exercise the rest of the generic kernel: several column slices,
ragged last chunks, chunk 1, T < chunk, T = 0, packed sequences including
empty ones, grouped heads, bf16 inputs, and in-place states.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import gpu_prefill, oracle_prefill, rel_err, say, dev

pytestmark = pytest.mark.gpu
TOL = 1e-4


def test_tiny_f32_workload():
    w = synth.WORKLOADS["tiny_f32"]
    inp = synth.workload_inputs(w)
    say("tiny_f32", w)
    out, hf, route = gpu_prefill(inp, w.chunk)
    assert route.startswith("gdn_prefill_generic_kernel grid=[1,1,1]"), route
    ro, rh = oracle_prefill(inp)
    eo, eh = rel_err(out, ro), rel_err(hf, rh)
    say(f"  out err {eo:.3e}  state err {eh:.3e}")
    assert eo <= TOL
    assert eh <= TOL


CASES = [
    # B, T, Hk, Hv, dk, dv, chunk, h0
    (2, 100, 2, 6, 24, 40, 16, True),
    (1, 77, 1, 2, 128, 128, 64, True),
    (1, 5, 1, 1, 16, 16, 64, True),
    (1, 64, 1, 1, 8, 8, 1, True),
    (2, 65, 1, 3, 32, 32, 64, False),
    (1, 200, 4, 8, 64, 16, 7, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_T%d_Hk%d_Hv%d_dk%d_dv%d_C%d_h%d" % c)
def test_generic_f32_shapes(case):
    B, T, Hk, Hv, dk, dv, C, h0 = case
    inp = synth.prefill_inputs(B, T, Hk, Hv, dk, dv, io=torch.float32, h0=h0, seed=7 + T)
    say("generic f32", case)
    out, hf, route = gpu_prefill(inp, C)
    assert "generic" in route, route
    ro, rh = oracle_prefill(inp)
    assert rel_err(out, ro) <= TOL
    assert rel_err(hf, rh) <= TOL


def test_generic_empty_sequence_keeps_state():
    inp = synth.prefill_inputs(3, 0, 1, 2, 16, 16, io=torch.float32, h0=True, seed=3)
    say("generic T=0")
    out, hf, _ = gpu_prefill(inp, 16)
    assert out.numel() == 0
    assert torch.equal(hf.cpu(), inp["h0"])


def test_generic_packed():
    lens = [37, 0, 64, 1, 100]
    inp = synth.prefill_inputs(len(lens), 0, 2, 4, 32, 48, io=torch.float32, h0=True, seed=11,
                               lengths=lens)
    say("generic packed", lens)
    out, hf, _ = gpu_prefill(inp, 32)
    ro, rh = oracle_prefill(inp)
    assert rel_err(out, ro) <= TOL
    assert rel_err(hf, rh) <= TOL
    assert torch.equal(hf[1].cpu(), inp["h0"][1])  # the empty sequence


def test_generic_bf16_inputs():
    inp = synth.prefill_inputs(1, 150, 2, 4, 64, 64, io=torch.bfloat16, h0=True, seed=12)
    say("generic bf16 in, f32 out")
    out, hf, route = gpu_prefill(inp, 32, out_dtype=torch.float32)
    assert "generic" in route
    ro, rh = oracle_prefill(inp)
    assert rel_err(out, ro) <= TOL
    assert rel_err(hf, rh) <= TOL


def test_generic_in_place_state():
    inp = synth.prefill_inputs(2, 50, 1, 2, 32, 32, io=torch.float32, h0=True, seed=13)
    g = {k: (v.to(dev()) if torch.is_tensor(v) else v) for k, v in inp.items()}
    h = g["h0"].clone()
    import linear_attention_ssm_gated_amd as gdn
    out = torch.empty_like(g["v"])
    say("generic in place")
    gdn.gdn_chunk_prefill(g["q"], g["k"], g["v"], g["log_g"], g["beta"], h, out, h,
                          2, 50, 1, 2, 32, 32, 16)
    torch.cuda.synchronize()
    ro, rh = oracle_prefill(inp)
    assert rel_err(h, rh) <= TOL
    assert rel_err(out, ro) <= TOL
