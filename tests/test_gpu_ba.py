"""GPU parity of the gate/beta producer (the BA projection) against the fp64
oracle: max|d|/max|ref| <= 1e-4 on the gates and on the betas (bf16 inputs,
fp32 accumulation and gating).

The full-size workload (4576 tokens, k = 5120, 2 x 48 outputs in groups of 3)
runs through the same entry point and launch configuration bench.py times,
every token checked.  Edge cases: 1, 63, 65, 130 and 200 tokens (partial
64-token tiles), k from 64 (one block, one split) to 5120, 1 to 4 v-heads per
group, n = 128 (eight output tiles), row strides wider than k (the extra
columns hold data and must be ignored), an output stride wider than 2 nv (the
padding must stay untouched), m = 0, and a repeated call (bitwise equal).
"""
import pytest
import torch

import linear_attention_ssm_gated_amd as gdn
import oracle
import synth
from gpu_common import dev, say

pytestmark = pytest.mark.gpu
TOL = 1e-4


def run(inp, nv, G, gate_stride=None, fill=float("nan")):
    d = dev()
    x, w = inp["x"].to(d), inp["w"].to(d)
    a_log, dt_bias = inp["a_log"].to(d), inp["dt_bias"].to(d)
    m, ks = x.shape
    n, k = w.shape
    gs = 2 * nv if gate_stride is None else gate_stride
    out = torch.full((m, gs), fill, dtype=torch.float32, device=d)
    ws = torch.empty(max(1, gdn.gdn_ba_gates_workspace_bytes(m, n, k)), dtype=torch.uint8, device=d)
    route = gdn.gdn_ba_gates(x, w, a_log, dt_bias, out, m, n, k, ks, gs, nv, G, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu(), route


def check(inp, nv, G, out):
    ref = oracle.ba_gates(inp["x"], inp["w"], inp["a_log"], inp["dt_bias"], nv, G)
    got = out[:, : 2 * nv].double().numpy()
    eg = synth.max_rel_err(got[:, :nv], ref[:, :nv])
    eb = synth.max_rel_err(got[:, nv:], ref[:, nv:])
    say(f"  gate err {eg:.3e}  beta err {eb:.3e}")
    assert eg <= TOL and eb <= TOL
    return eg, eb


def test_full_workload_every_token():
    wl = synth.BA_WORKLOAD
    inp = synth.ba_inputs(wl["m"], wl["k"], wl["nv"], seed=wl["seed"])
    say(wl["name"])
    out, route = run(inp, wl["nv"], wl["vheads_per_group"])
    assert route.startswith("gdn_ba_partial_kernel+gdn_ba_gate_kernel"), route
    check(inp, wl["nv"], wl["vheads_per_group"], out)


@pytest.mark.parametrize("m,k,nv,G,xpad,opad", [
    (1, 64, 1, 1, 0, 0),
    (63, 128, 4, 2, 8, 3),
    (65, 192, 6, 3, 16, 0),
    (130, 5120, 48, 3, 0, 5),
    (200, 640, 64, 4, 24, 1),
    (77, 320, 12, 1, 0, 0),
])
def test_shapes(m, k, nv, G, xpad, opad):
    inp = synth.ba_inputs(m, k, nv, seed=400 + m, x_stride=k + xpad)
    say("ba shape", m, k, nv, G, xpad, opad)
    out, _ = run(inp, nv, G, gate_stride=2 * nv + opad)
    check(inp, nv, G, out)
    if opad:
        assert torch.isnan(out[:, 2 * nv:]).all(), "padding of the output row changed"


def test_zero_tokens_is_a_no_op():
    say("ba m = 0")
    d = dev()
    w = torch.zeros((96, 5120), dtype=torch.bfloat16, device=d)
    route = gdn.gdn_ba_gates(None, w, None, None, None, 0, 96, 5120, 5120, 96, 48, 3, workspace=None)
    assert route.startswith("gdn_ba_partial_kernel")


def test_repeat_is_bitwise_equal():
    inp = synth.ba_inputs(500, 1024, 16, seed=401)
    say("ba determinism")
    o1, _ = run(inp, 16, 4)
    o2, _ = run(inp, 16, 4)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))


def test_gates_feed_the_prefill():
    # the producer's [gate | beta] row, split into log_g and beta, drives a
    # prefill: its outputs equal the oracle prefill run on the oracle's gates
    m, k, nv, G = 300, 256, 6, 3
    Hk = nv // G
    inp = synth.ba_inputs(m, k, nv, seed=402)
    say("ba -> prefill")
    out, _ = run(inp, nv, G)
    pre = synth.prefill_inputs(1, m, Hk, nv, 128, 128, h0=True, seed=403)
    ref_gates = oracle.ba_gates(inp["x"], inp["w"], inp["a_log"], inp["dt_bias"], nv, G)
    d = dev()
    log_g = out[:, :nv].contiguous().reshape(1, m, nv)
    beta = out[:, nv:].contiguous().reshape(1, m, nv)
    o, hf, _ = gdn.chunk_prefill(pre["q"].to(d), pre["k"].to(d), pre["v"].to(d), log_g.to(d), beta.to(d),
                                 pre["h0"].to(d), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rh = oracle.prefill(pre["q"], pre["k"], pre["v"], ref_gates[:, :nv].reshape(1, m, nv),
                            ref_gates[:, nv:].reshape(1, m, nv), pre["h0"])
    eo = synth.max_rel_err(o.double().cpu().numpy(), ro)
    eh = synth.max_rel_err(hf.double().cpu().numpy(), rh)
    say(f"  prefill out err {eo:.3e} state err {eh:.3e}")
    assert eo <= 2e-2 and eh <= 2e-2
