"""GPU parity of the segment-scan prefill (gdn_chunk_prefill_segmented)
against the fp64 oracle, at the bar of the plain MFMA prefill: max|d|/max|ref|
<= 2e-2 on outputs and final states.

The segment scan is taken for dense input whose spine workgroups fill at most
a third of the chip; each sequence is cut into chunk-aligned segments whose
affine state maps are combined in order.  Checks:
  * slowly decaying gates (the synthetic gates forget the start of a
    512-token segment below fp32 resolution, so they alone would leave the
    combined maps untested) and the workload's own gates;
  * the narrow 4576-token workload (6 v-heads over 2 k-heads) on every v-head,
    and against the plain spine's result on the same input;
  * ragged tails, no initial state, fp32 outputs, two sequences, no final
    state, and the final state written over the initial one (in place);
  * two runs give the same bytes;
  * the cut itself (segments and chunks per segment) from the route's grid;
  * packed input and wide layers fall back to the plain spine and say why.
"""
import pytest
import torch

import linear_attention_ssm_gated_amd as gdn
import synth
from gpu_common import dev, gpu_prefill, oracle_prefill, rel_err, say

pytestmark = pytest.mark.gpu
TOL = 2e-2
SEG = ("gdn_wy_prep_kernel+gdn_spine_kernel(segment maps)+gdn_segment_combine_kernel"
       "+gdn_spine_kernel(segment outputs)")
PLAIN = "gdn_wy_prep_kernel+gdn_spine_kernel grid="


def expected_cut(B, T, Hv):
    """Segments per sequence of the cut: the most whose map walks (2 S - 3
    per sequence, v-head and 32-column tile) fit in 256 workgroups, whole
    chunks per segment."""
    nc = (T + 63) // 64
    s0 = min(nc, (256 // (B * Hv * 4) + 3) // 2, 10)
    L = -(-nc // s0)
    return -(-nc // L)


def check(inp, out, hf):
    ro, rh = oracle_prefill(inp)
    eo = rel_err(out, ro)
    eh = rel_err(hf, rh, head_axis=1)
    say(f"  out err {eo:.3e}  state err {eh:.3e}")
    assert eo <= TOL
    assert eh <= TOL


def test_narrow_workload_all_heads():
    w = synth.WORKLOADS["prefill_t4576_hv6"]
    inp = synth.workload_inputs(w)
    say(w.name, "segmented")
    out, hf, route = gpu_prefill(inp, w.chunk, segmented=True)
    S = expected_cut(w.B, w.T, w.Hv)
    assert route.startswith(f"{SEG} grid=[{w.Hv * 4},{w.B * S},1]"), route
    check(inp, out, hf)
    say(w.name, "again, bytes compared")
    out2, hf2, _ = gpu_prefill(inp, w.chunk, segmented=True)
    assert torch.equal(out, out2) and torch.equal(hf, hf2), "two runs give the same bytes"


def test_slow_gates_against_the_plain_spine():
    """The narrow workload's shape with gates 50x slower (a mean decay of
    about 0.0016 per token): the start states carry across segments."""
    inp = synth.prefill_inputs(1, 4576, 2, 6, 128, 128, h0=True, seed=1110, gate_scale=0.002)
    say("slow gates, segmented")
    out, hf, route = gpu_prefill(inp, 64, segmented=True)
    assert route.startswith(SEG), route
    check(inp, out, hf)
    say("slow gates, plain spine")
    out_p, hf_p, route_p = gpu_prefill(inp, 64)
    assert route_p.startswith(PLAIN), route_p
    d_out = rel_err(out, out_p.float().cpu().double().numpy())
    d_state = rel_err(hf, hf_p.cpu().double().numpy(), head_axis=1)
    say(f"  segment scan vs plain spine: out {d_out:.3e}  state {d_state:.3e}")
    assert 0 < d_state <= TOL and d_out <= TOL


@pytest.mark.parametrize("B,T,Hk,Hv,h0,f32,gs", [
    (2, 64 * 37 + 5, 1, 3, True, False, 0.002),    # ragged last segment, two sequences
    (1, 64 * 40, 1, 2, False, False, 0.002),       # no initial state, every segment full
    (1, 64 * 12 + 63, 2, 4, True, True, 0.002),    # fp32 outputs, two-chunk segments
    (1, 64 * 3, 1, 1, True, False, 0.1),           # three segments of one chunk each
    (1, 64 * 9 + 1, 1, 6, True, False, 0.0),       # no decay at all; a one-row last chunk
])
def test_cuts(B, T, Hk, Hv, h0, f32, gs):
    inp = synth.prefill_inputs(B, T, Hk, Hv, 128, 128, h0=h0, seed=1100 + T + Hv, gate_scale=gs)
    say("segment scan", B, T, Hk, Hv, h0, f32, gs)
    out, hf, route = gpu_prefill(inp, 64, out_dtype=torch.float32 if f32 else None, segmented=True)
    S = expected_cut(B, T, Hv)
    assert S >= 3
    assert route.startswith(f"{SEG} grid=[{Hv * 4},{B * S},1]"), route
    check(inp, out, hf)


def test_without_final_state():
    """h_final NULL: the output walks still run from the combined start states."""
    inp = synth.prefill_inputs(1, 64 * 20 + 17, 1, 3, 128, 128, h0=True, seed=1150, gate_scale=0.002)
    say("segment scan, no final state")
    out, hf, route = gpu_prefill(inp, 64, want_state=False, segmented=True)
    assert hf is None and route.startswith(SEG), route
    ro, _ = oracle_prefill(inp)
    e = rel_err(out, ro)
    say(f"  out err {e:.3e}")
    assert e <= TOL


def test_in_place_state():
    """h_final aliasing h0, as the plain route allows: the last segment's
    walk writes the final state while segment 0's walk starts from h0."""
    B, T, Hk, Hv = 2, 64 * 30 + 9, 1, 3
    inp = synth.prefill_inputs(B, T, Hk, Hv, 128, 128, h0=True, seed=1160, gate_scale=0.002)
    g = {k: (v.to(dev()) if torch.is_tensor(v) else v) for k, v in inp.items()}
    h = g["h0"].clone()
    out = torch.empty_like(g["v"])
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(B, T, Hk, Hv, 128, 128, 64, gdn.GDN_BF16),
                     dtype=torch.uint8, device=dev())
    say("segment scan in place")
    route = gdn.gdn_chunk_prefill_segmented(g["q"], g["k"], g["v"], g["log_g"], g["beta"], h, out, h,
                                            B, T, Hk, Hv, 128, 128, 64, workspace=ws)
    torch.cuda.synchronize()
    assert route.startswith(SEG), route
    check(inp, out, h)


def test_falls_back_to_the_plain_spine():
    inp = synth.prefill_inputs(2, 0, 1, 2, 128, 128, h0=True, seed=1201, lengths=[300, 700])
    say("segment scan refused: packed")
    out, hf, route = gpu_prefill(inp, 64, segmented=True)
    assert route.startswith(PLAIN) and "takes dense input" in route, route
    check(inp, out, hf)
    inp = synth.prefill_inputs(1, 700, 4, 24, 128, 128, h0=True, seed=1202)
    say("segment scan refused: 96 spine workgroups")
    out, hf, route = gpu_prefill(inp, 64, segmented=True)
    assert route.startswith(PLAIN) and "fill the chip" in route, route
    ro, rh = oracle_prefill(inp, heads=[0, 23])
    assert rel_err(out, ro, heads=[0, 23]) <= TOL
