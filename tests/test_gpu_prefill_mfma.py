"""GPU parity of the bf16 MFMA chunked prefill (dk = dv = 128, chunk 64)
against the fp64 oracle: max|d|/max|ref| <= 2e-2 on outputs and final states
(bf16 MFMA operands, fp32 accumulators and state).

Full-size workloads run through the same entry point and launch
configuration bench.py times: the 1168-token and 4576-token calls and the
packed 8-sequence workload are checked on every v-head.
Edge cases: sequences of 1, 63, 64, 65 and 130 tokens, empty packed
sequences, fp32 outputs, in-place states, and 1, 2, 4, 5 and 8 v-heads per
k-head (the WY kernel runs one wave per v-head in groups of up to four, so 5
leaves a partial last group).  Bitwise properties: repeated runs,
a state carried across a chunk-aligned split, packed vs separate runs, and
the Q rows brought in by either wave (the recurrence waves in a launch of 192
or more workgroups that writes outputs, the loader otherwise).
"""
import numpy as np
import pytest
import torch

import linear_attention_ssm_gated_amd as gdn
import synth
from gpu_common import dev, gpu_prefill, oracle_prefill, rel_err, say

pytestmark = pytest.mark.gpu
TOL = 2e-2
ROUTE = "gdn_wy_prep_kernel+gdn_spine_kernel"


def check(inp, out, hf, heads=None):
    ro, rh = oracle_prefill(inp, heads=heads)
    eo = rel_err(out, ro, heads=heads)
    eh = rel_err(hf, rh, heads=heads, head_axis=1)
    say(f"  out err {eo:.3e}  state err {eh:.3e}")
    assert eo <= TOL
    assert eh <= TOL
    return eo, eh


@pytest.mark.parametrize("name", ["prefill_t1168", "prefill_t4576_h0"])
def test_full_workload_all_heads(name):
    w = synth.WORKLOADS[name]
    inp = synth.workload_inputs(w)
    say(name)
    out, hf, route = gpu_prefill(inp, w.chunk)
    assert route.startswith(ROUTE), route
    check(inp, out, hf)


def test_packed_workload_all_heads():
    """The packed 8-sequence workload (28,946 tokens, up to 6,604 in one
    sequence) on every v-head; the longest sequence's own error is reported."""
    w = synth.WORKLOADS["varlen_b8"]
    inp = synth.workload_inputs(w)
    cu = inp["cu_seqlens"].tolist()
    say("varlen_b8", cu)
    out, hf, route = gpu_prefill(inp, w.chunk)
    assert route.startswith(ROUTE), route
    ro, rh = oracle_prefill(inp)
    eo = rel_err(out, ro)
    eh = rel_err(hf, rh, head_axis=1)
    lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    b = int(np.argmax(lens))
    eo_b = rel_err(out[cu[b]:cu[b + 1]], ro[cu[b]:cu[b + 1]])
    eh_b = rel_err(hf[b], rh[b])
    say(f"  all heads: out err {eo:.3e}  state err {eh:.3e}; longest sequence ({lens[b]} tokens): "
        f"out err {eo_b:.3e}  state err {eh_b:.3e}")
    assert eo <= TOL and eh <= TOL


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_short_and_ragged(T):
    inp = synth.prefill_inputs(2, T, 1, 3, 128, 128, h0=True, seed=100 + T)
    say("ragged", T)
    out, hf, route = gpu_prefill(inp, 64)
    assert route.startswith(ROUTE)
    check(inp, out, hf)


@pytest.mark.parametrize("Hk,Hv", [(3, 3), (2, 4), (1, 4), (2, 10), (1, 8)])
def test_vheads_per_khead(Hk, Hv):
    inp = synth.prefill_inputs(1, 150, Hk, Hv, 128, 128, h0=True, seed=200 + 10 * Hk + Hv)
    say("v-heads per k-head", Hk, Hv)
    out, hf, route = gpu_prefill(inp, 64)
    assert route.startswith(ROUTE)
    check(inp, out, hf)


def test_packed_with_empty_and_short_sequences():
    lens = [1, 0, 64, 65, 200, 0]
    inp = synth.prefill_inputs(len(lens), 0, 2, 4, 128, 128, h0=True, seed=31, lengths=lens)
    say("packed edge", lens)
    out, hf, _ = gpu_prefill(inp, 64)
    check(inp, out, hf)
    for b in (1, 5):
        assert torch.equal(hf[b].cpu(), inp["h0"][b]), "an empty sequence keeps its state"


def test_packed_dispatch_order_up_to_and_past_256_sequences():
    # the spine walks packed sequences longest first when there are at most
    # 256 of them, in index order past that; either way every sequence's
    # result is its own: equal to the oracle, and equal bit for bit to the
    # same sequences packed in reverse
    for B in (40, 300):
        rng = np.random.default_rng(900 + B)
        lens = [int(x) for x in rng.integers(0, 150, size=B)]
        lens[B // 2] = 700                     # one long walk in the middle
        inp = synth.prefill_inputs(B, 0, 1, 2, 128, 128, h0=True, seed=901 + B, lengths=lens)
        say("packed dispatch order", B, sum(lens))
        out, hf, _ = gpu_prefill(inp, 64)
        check(inp, out, hf, heads=[0, 1])
        # the same sequences packed in reverse order
        cu = inp["cu_seqlens"].tolist()
        rev = {}
        for key in ("q", "k", "v", "log_g", "beta"):
            t = inp[key]
            rev[key] = torch.cat([t[cu[b]:cu[b + 1]] for b in reversed(range(B))], dim=0)
        rev["h0"] = torch.flip(inp["h0"], dims=[0]).contiguous()
        rl = list(reversed(lens))
        rev["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(rl)]), dtype=torch.int32)
        out_r, hf_r, _ = gpu_prefill(rev, 64)
        cr = rev["cu_seqlens"].tolist()
        for b in range(B):
            rb = B - 1 - b
            assert torch.equal(_bits(out[cu[b]:cu[b + 1]]), _bits(out_r[cr[rb]:cr[rb + 1]])), (B, b)
            assert torch.equal(_bits(hf[b]), _bits(hf_r[rb])), (B, b)


def test_fp32_output_and_no_initial_state():
    inp = synth.prefill_inputs(1, 300, 2, 6, 128, 128, h0=False, seed=32)
    say("fp32 out")
    out, hf, _ = gpu_prefill(inp, 64, out_dtype=torch.float32)
    assert out.dtype == torch.float32
    check(inp, out, hf)


def test_in_place_state():
    inp = synth.prefill_inputs(2, 150, 1, 3, 128, 128, h0=True, seed=33)
    g = {k: (v.to(dev()) if torch.is_tensor(v) else v) for k, v in inp.items()}
    h = g["h0"].clone()
    out = torch.empty_like(g["v"])
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(2, 150, 1, 3, 128, 128, 64, gdn.GDN_BF16),
                     dtype=torch.uint8, device=dev())
    say("in place")
    gdn.gdn_chunk_prefill(g["q"], g["k"], g["v"], g["log_g"], g["beta"], h, out, h,
                          2, 150, 1, 3, 128, 128, 64, workspace=ws)
    torch.cuda.synchronize()
    check(inp, out, h)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_deterministic():
    inp = synth.prefill_inputs(1, 700, 2, 6, 128, 128, h0=True, seed=34)
    say("determinism")
    o1, h1, _ = gpu_prefill(inp, 64)
    o2, h2, _ = gpu_prefill(inp, 64)
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(h1), _bits(h2))


def test_state_carry_is_bitwise_at_chunk_boundary():
    T1, T2 = 128, 150
    inp = synth.prefill_inputs(1, T1 + T2, 2, 6, 128, 128, h0=True, seed=35)
    part = lambda sl: {k: (v[:, sl].contiguous() if k in ("q", "k", "v", "log_g", "beta") else v)
                       for k, v in inp.items()}
    say("carry")
    o, h, _ = gpu_prefill(inp, 64)
    o1, h1, _ = gpu_prefill(part(slice(0, T1)), 64)
    o2, h2, _ = gpu_prefill(part(slice(T1, None)), 64, h0=h1)
    assert torch.equal(_bits(torch.cat([o1, o2], dim=1)), _bits(o))
    assert torch.equal(_bits(h2), _bits(h))


def test_packed_equals_separate_bitwise():
    lens = [70, 129, 5]
    inp = synth.prefill_inputs(len(lens), 0, 1, 3, 128, 128, h0=True, seed=36, lengths=lens)
    say("packed vs separate")
    out, hf, _ = gpu_prefill(inp, 64)
    cu = inp["cu_seqlens"].tolist()
    for b, L in enumerate(lens):
        sl = slice(cu[b], cu[b + 1])
        one = {k: (v[sl].unsqueeze(0).contiguous() if k in ("q", "k", "v", "log_g", "beta") else v)
               for k, v in inp.items()}
        one["h0"] = inp["h0"][b : b + 1]
        one["cu_seqlens"] = None
        o, h, _ = gpu_prefill(one, 64)
        assert torch.equal(_bits(o[0]), _bits(out[sl])), b
        assert torch.equal(_bits(h[0]), _bits(hf[b])), b


def test_q_rows_from_either_wave_bitwise():
    """Two dense sequences of 24 v-heads in one call (grid 96 x 2 = 192
    workgroups: the recurrence waves issue the Q rows) against each sequence
    alone (96 workgroups: the loader issues them): the same bits."""
    B, T, Hk, Hv = 2, 64 * 6 + 17, 8, 24
    inp = synth.prefill_inputs(B, T, Hk, Hv, 128, 128, h0=True, seed=37)
    say("Q rows by the recurrence waves vs by the loader")
    out, hf, route = gpu_prefill(inp, 64)
    assert route.startswith(f"{ROUTE} grid=[{Hv * 4},{B},1]"), route
    check(inp, out, hf)
    for b in range(B):
        one = {k: (v[b : b + 1].contiguous() if torch.is_tensor(v) else v) for k, v in inp.items()}
        o, h, r1 = gpu_prefill(one, 64)
        assert r1.startswith(f"{ROUTE} grid=[{Hv * 4},1,1]"), r1
        assert torch.equal(_bits(o[0]), _bits(out[b])), b
        assert torch.equal(_bits(h[0]), _bits(hf[b])), b


@pytest.mark.parametrize("scale", [30.0, 200.0])
def test_strong_gates(scale):
    """Gates far stronger than the synthetic ones: log_g scaled by 30 (about -150
    per 64-token chunk) and by 200 (about -1000 per chunk, decay underflows to
    zero within a chunk).  Every decay factor the kernels form is exp of a
    non-positive difference, so nothing overflows: outputs and states stay
    finite and match the oracle."""
    inp = synth.prefill_inputs(1, 300, 2, 6, 128, 128, h0=True, seed=903)
    inp["log_g"] = inp["log_g"] * scale
    say("strong gates x", scale)
    out, hf, route = gpu_prefill(inp, 64)
    assert route.startswith(ROUTE)
    assert torch.isfinite(out.float()).all() and torch.isfinite(hf).all()
    check(inp, out, hf)


def test_gates_from_the_ba_producer():
    """The gate/beta producer's output (strongly decaying gates: chunk sums down
    to about -114 on some v-heads) feeding the prefill, checked against the
    oracle on the same gates."""
    import linear_attention_ssm_gated_amd as gdn_
    T, Hk, Hv, kdim = 320, 2, 6, 512
    ba = synth.ba_inputs(T, kdim, Hv, seed=1006)
    x, w = ba["x"].to(dev()), ba["w"].to(dev())
    gates, _ = gdn_.ba_gates(x, w, ba["a_log"].to(dev()), ba["dt_bias"].to(dev()), Hv, Hv // Hk)
    torch.cuda.synchronize()
    inp = synth.prefill_inputs(1, T, Hk, Hv, 128, 128, h0=True, seed=904)
    g = gates.cpu()
    inp["log_g"] = g[:, :Hv].reshape(1, T, Hv).contiguous()
    inp["beta"] = g[:, Hv:].reshape(1, T, Hv).contiguous()
    sums = inp["log_g"][0, :256].reshape(4, 64, Hv).sum(1)
    say("ba gates: min chunk sum", float(sums.min()))
    out, hf, route = gpu_prefill(inp, 64)
    assert route.startswith(ROUTE)
    assert torch.isfinite(out.float()).all() and torch.isfinite(hf).all()
    check(inp, out, hf)
