"""The entry points captured into a HIP graph, as bench.py times them: each
replay must give the eager call's bytes.  Replays run three times with the
program's own eager work and synchronisations between them, and every replay
is checked (kernels only; no memset nodes are recorded).
"""
import pytest
import torch

import linear_attention_ssm_gated_amd as gdn
import synth
from gpu_common import dev, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                          # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fn()
    torch.cuda.synchronize()
    return g


def _replays(fn, outs, n=3):
    """Eager reference bytes, then n replays of a captured graph of fn, each
    compared with the reference; eager work of the program in between."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = _capture(fn)
    for r in range(n):
        for o in outs:
            o.fill_(0)               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(_bits(o), _bits(e)), f"replay {r} differs from the eager call"


def test_prefill_graph_replay():
    d = dev()
    inp = synth.prefill_inputs(1, 700, 2, 6, 128, 128, h0=True, seed=500)
    g = {k: (v.to(d) if torch.is_tensor(v) else v) for k, v in inp.items()}
    out = torch.empty_like(g["v"])
    hf = torch.empty((1, 6, 128, 128), dtype=torch.float32, device=d)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(1, 700, 2, 6, 128, 128, 64, gdn.GDN_BF16),
                     dtype=torch.uint8, device=d)
    say("graph replay: prefill")

    def fn():
        gdn.gdn_chunk_prefill(g["q"], g["k"], g["v"], g["log_g"], g["beta"], g["h0"], out, hf,
                              1, 700, 2, 6, 128, 128, 64, workspace=ws)
    _replays(fn, [out, hf])


def test_verify_graph_replay():
    d = dev()
    B, K, Hk, Hv = 4, 4, 2, 6
    di = synth.decode_inputs(B, K, Hk, Hv, 128, 128, seed=501)
    states = [di["states"][b].to(d).clone() for b in range(B)]
    table = torch.tensor([s.data_ptr() for s in states], dtype=torch.int64, device=d)
    q = di["q"].reshape(B * K, -1).to(d)
    k = di["k"].reshape(B * K, -1).to(d)
    v = di["v"].reshape(B * K, -1).to(d)
    gate = di["gate"].reshape(B * K, -1).to(d)
    beta = di["beta"].reshape(B * K, -1).to(d)
    out = torch.empty((B, K, Hv, 128), dtype=torch.bfloat16, device=d)
    ssf = gdn.gdn_stash_seq_floats(Hv, 128, 128, K, gdn.GDN_BF16)
    stash = torch.empty(B * ssf, dtype=torch.float32, device=d)
    flag = torch.zeros(1, dtype=torch.int32, device=d)
    say("graph replay: verify")

    def fn():   # the verify writes no state, so every replay sees the same inputs
        gdn.gdn_flag_clear(flag)
        gdn.gdn_decode_verify_k4(table, q, k, v, gate, beta, out, stash, B, Hk, Hv, 128, 128,
                                 Hk * 128, Hv * 128, Hv, ssf, flag)
    _replays(fn, [out, stash, flag])


def test_ba_gates_graph_replay():
    d = dev()
    m, k, nv, G = 600, 1024, 48, 3
    inp = synth.ba_inputs(m, k, nv, seed=502)
    x, w = inp["x"].to(d), inp["w"].to(d)
    a_log, dt_bias = inp["a_log"].to(d), inp["dt_bias"].to(d)
    out = torch.empty((m, 2 * nv), dtype=torch.float32, device=d)
    ws = torch.empty(gdn.gdn_ba_gates_workspace_bytes(m, 2 * nv, k), dtype=torch.uint8, device=d)
    say("graph replay: ba gates")

    def fn():
        gdn.gdn_ba_gates(x, w, a_log, dt_bias, out, m, 2 * nv, k, k, 2 * nv, nv, G, workspace=ws)
    _replays(fn, [out])
