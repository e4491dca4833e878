"""Throughput of the gated delta rule chunked prefill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one gdn_chunk_prefill call (the whole hot path: WY terms, state
spine, chunk outputs, final states) over one batch of synthetic inputs that
already sit in HBM.  The default workload is one 4576-token sequence with 48
v-heads over 16 k-heads, d = 128, chunk 64, bf16 q/k/v, fp32 gates, an fp32
initial state and fp32 final states.  Inputs rotate over enough copies
(> 512 MB in total) that the 256 MB Infinity Cache cannot hold them between
steps.  Prints one JSON line; the default run adds the K = 4 verify's and the
fold's HBM rooflines and the 6-v-head share of the layer (plain spine and
segment scan) as extra keys.  Other workloads: prefill_t1168,
varlen_b8 and prefill_t4576_hv6 (prefill, tokens/s; --segmented times
gdn_chunk_prefill_segmented), verify_k4_b16, step_b16 and ba_gates_t4576
(HBM-bound; metric GB/s).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
ROTATE_BYTES = 600e6        # > 2 x 256 MB Infinity Cache
DEFAULT_WORKLOAD = "prefill_t4576_h0"


# ---- accounting: algorithmic work of the method (not of any kernel) --------

def prefill_bytes(lengths, Hk, Hv, dk, dv, s_io=2, s_out=2, h0=True, h_final=True):
    """Compulsory HBM bytes: read q, k, v, log_g, beta once, write out once,
    read h0 and write h_final once per (sequence, v-head)."""
    N = sum(lengths)
    per_token = 2 * Hk * dk * s_io + Hv * dv * s_io + 8 * Hv + Hv * dv * s_out
    per_seq = Hv * dk * dv * 4 * (int(h0) + int(h_final))
    return N * per_token + len(lengths) * per_seq


def prefill_flops(lengths, Hk, Hv, dk, dv, chunk):
    """2 x MACs the chunked method needs, per chunk of L rows and v-head:
    3 L dk dv (W h, K~^T Delta, Q h) + L(L+1)/2 (dk + 2 dv) (W, U, P Delta)
    + L^3/6 (UT solve) + (Hk/Hv) L^2 dk (K K^T and Q K^T, shared by the
    v-heads of one k-head)."""
    mac = 0.0
    for T in lengths:
        for t0 in range(0, T, chunk):
            L = min(chunk, T - t0)
            mac += 3 * L * dk * dv + L * (L + 1) / 2 * (dk + 2 * dv) + L ** 3 / 6 + (Hk / Hv) * L * L * dk
    return 2 * mac * Hv


def verify_bytes(B, Hk, Hv, dk, dv, s_io=2, s_out=2, K=4):
    """Read each state once, the K rows of q, k, v, gate, beta; write the K
    outputs and the stash (delta fp32, G fp32, keys bf16)."""
    return (B * Hv * dk * dv * 4 + B * K * (2 * Hk * dk + Hv * dv) * s_io + B * K * Hv * 8
            + B * K * Hv * dv * s_out + B * Hv * (K * dv * 4 + K * 4 + K * dk * 2))


def fold_bytes(na, Hv, dk, dv, K=4):
    """Per sequence with na > 0 and v-head: read and write the state once, read
    the na stashed rows (delta fp32, key bf16) and G."""
    return sum(Hv * (2 * dk * dv * 4 + n * (dv * 4 + dk * 2) + K * 4) for n in na if n > 0)


def step_bytes(B, Hk, Hv, dk, dv, s_io=2, s_out=2):
    """Read and write each state once; read one row of q, k, v, gate, beta per
    sequence; write one output row."""
    return (B * Hv * dk * dv * 4 * 2 + B * (2 * Hk * dk + Hv * dv) * s_io + B * Hv * 8
            + B * Hv * dv * s_out)


def ba_bytes(m, k, nv):
    """Read the activations, the weight and the two parameter vectors once;
    write the [gate | beta] rows once."""
    return m * k * 2 + 2 * nv * k * 2 + 2 * nv * 4 + m * 2 * nv * 4


def kernel_source_sha():
    import glob
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "linear_attention_ssm_gated_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    return rec.get("bytes_per_launch")


def measured_kernel_traffic(name, kernel):
    """HBM bytes (read + write) of one kernel of a profiled workload, under the
    same conditions as measured_traffic; else None."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    k = rec.get("per_kernel_bytes", {}).get(kernel)
    return None if k is None else k["read"] + k["write"]


# ---- timing ----------------------------------------------------------------

def time_launches(launch, n_sets, warmup, steps, torch, extra_replays=10):
    """Warm up, then time `steps` launches (rotating input sets) with HIP events.

    The timed launches are captured into one HIP graph and the graph is replayed
    between two events on the replay stream, so the kernels run back to back as
    under a serving loop; eagerly, the Python launch path (tens of microseconds
    per call) would leave the GPU idle between short kernels.  The graph is
    replayed 1 + `extra_replays` times, each replay timed on its own (exactly
    `steps` launches between its events, synchronized before and after); the
    measurement is the median replay.  The first timed replay runs up to ~8%
    slower than the rest for the short decode kernels (the clocks settle again
    after each host synchronization), so a single replay would report that
    transient rather than the steady state a serving loop sees; it stays in the
    spread as `first_replay_us`.  Returns (median replay ms, median ms per
    launch, eager ms per launch, spread), the third from an event pair around
    each of `steps` eager launches, for reference."""
    for i in range(warmup):
        launch(i % n_sets)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        launch(i % n_sets)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    eager = sum(a.elapsed_time(b) for a, b in ev) / steps
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                launch(i % n_sets)
    torch.cuda.synchronize()
    # untimed: the first replay uploads the graph
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    per = []
    for _ in range(1 + extra_replays):
        torch.cuda.synchronize()
        t0.record(stream)
        graph.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        per.append(t0.elapsed_time(t1) / steps * 1e3)
    q = sorted(per)
    pick = lambda f: q[min(len(q) - 1, int(round(f * (len(q) - 1))))]
    med_us = pick(0.5)
    spread = {"median_us": med_us, "p10_us": pick(0.1), "p90_us": pick(0.9), "first_replay_us": per[0],
              "replays": len(q), "launches_per_replay": steps}
    return med_us * steps / 1e3, med_us / 1e3, eager, spread


def achievable_copy_gbs(torch, mib=1024, reps=10):
    """Bytes moved (read + write) per second by the runtime's own device-to-device
    copy of `mib` MiB, median of `reps`: the achievable-HBM yardstick beside the
    published peak."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        t0.record()
        dst.copy_(src)
        t1.record()
        torch.cuda.synchronize()
        ts.append(t0.elapsed_time(t1))
    ts.sort()
    del src, dst
    return 2 * n / (ts[len(ts) // 2] * 1e-3) / 1e9


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_prefill(inp, w, T, budget_s=10.0, max_reps=30):
    """The fp64 oracle on the whole workload, repeated until about budget_s of
    wall time has passed (at most max_reps runs)."""
    import oracle
    n = oracle.default_threads()
    reps = 0
    t = time.perf_counter()
    while True:
        oracle.prefill(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["beta"], inp["h0"], nthreads=n)
        reps += 1
        dt = time.perf_counter() - t
        if dt >= budget_s or reps >= max_reps:
            break
    return {"value": reps * T / dt, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"the whole workload ({T} tokens x {w.Hv} v-heads, fp64 token loop) {reps} times, "
                      f"{dt:.1f} s wall on {n} threads"}


def bench_prefill(w, args, torch):
    import linear_attention_ssm_gated_amd as gdn
    import synth
    d = torch.device("cuda:0")
    inp = synth.workload_inputs(w)
    if inp["cu_seqlens"] is not None:
        cu = inp["cu_seqlens"].tolist()
        lengths = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
        N = cu[-1]
    else:
        lengths = [w.T] * w.B
        N = w.B * w.T
    byt = prefill_bytes(lengths, w.Hk, w.Hv, w.dk, w.dv, h0=w.h0)
    flops = prefill_flops(lengths, w.Hk, w.Hv, w.dk, w.dv, w.chunk)
    n_sets = max(3, int(ROTATE_BYTES // byt) + 1)
    sets = []
    for i in range(n_sets):
        g = {k: (v.to(d) if torch.is_tensor(v) else v) for k, v in inp.items()}
        if g["h0"] is not None:
            g["h0"] = g["h0"].clone()
        g["out"] = torch.empty(g["v"].shape, dtype=torch.bfloat16, device=d)
        g["hf"] = torch.empty((w.B, w.Hv, w.dk, w.dv), dtype=torch.float32, device=d)
        sets.append(g)
    T_arg = N if inp["cu_seqlens"] is not None else w.T
    ws_n = gdn.gdn_prefill_workspace_bytes(w.B, T_arg, w.Hk, w.Hv, w.dk, w.dv, w.chunk, gdn.GDN_BF16,
                                           packed=inp["cu_seqlens"] is not None)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=d)
    route = []

    call = gdn.gdn_chunk_prefill_segmented if args.segmented else gdn.gdn_chunk_prefill

    def launch(i):   # on the current stream (the capture stream while a graph is recorded)
        g = sets[i]
        r = call(g["q"], g["k"], g["v"], g["log_g"], g["beta"], g["h0"], g["out"],
                 g["hf"], w.B, T_arg, w.Hk, w.Hv, w.dk, w.dv, w.chunk,
                 cu_seqlens=g["cu_seqlens"], workspace=ws, stream=None)
        if not route:
            route.append(r)

    total_ms, kern_ms, eager_ms, spread = time_launches(launch, n_sets, args.warmup, args.steps, torch)
    ms = total_ms / args.steps
    # parity of the timed launch's output on a few v-heads (fp64 oracle)
    import oracle
    heads = [0, w.Hv // 2, w.Hv - 1]
    ro, rh = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["beta"], inp["h0"],
                            cu_seqlens=None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy(),
                            heads=heads)
    import numpy as np
    got = sets[(args.steps - 1) % n_sets]["out"].float().cpu().numpy()
    err = synth.max_rel_err(np.take(got, heads, axis=-2), np.take(ro, heads, axis=-2))
    ach = byt / (kern_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name + ("_segmented" if args.segmented else ""))
    rec = {
        "metric": (f"GDN chunked-prefill tokens/s (Hv={w.Hv}, d={w.dk}, "
                   + (f"T={w.T}" if inp["cu_seqlens"] is None else f"{w.B} packed sequences, N={N}")
                   + "); % of MFMA/HBM peak"),
        "value": N / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "seed": w.seed, "B": w.B, "T": N, "Hk": w.Hk, "Hv": w.Hv, "dk": w.dk,
                   "dv": w.dv, "chunk": w.chunk, "h0": w.h0, "out": "bf16", "h_final": "fp32",
                   "entry": "gdn_chunk_prefill_segmented" if args.segmented else "gdn_chunk_prefill",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": byt, "algorithmic_flops": flops,
                     "mfma_tflops": flops / (kern_ms * 1e-3) / 1e12,
                     "mfma_frac": flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                     "fractions": {"hbm_bytes_of_8TBs": ach / HBM_PEAK_GBS,
                                   "mfma_flops_of_2500TFs": flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                   "note": "bound is hbm: at algorithmic bytes the call sits below the "
                                           "bf16 ridge (~181 of ~312 FLOP/B), so HBM is its roof; "
                                           "the target is stated as a fraction of MFMA peak"},
                     "kernel_ms": kern_ms, "eager_launch_ms": eager_ms, "spread": spread,
                     "kernel": route[0].split(" ")[0] if route else None},
        "timing": "median of 11 replays of a HIP graph of the K launches, HIP events around each replay",
        "route": route[0] if route else None,
        "parity_max_rel_err_sampled_heads": err,
        "input_sets_rotated": n_sets,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_prefill(inp, w, N)
    return rec


def bench_verify(w, args, torch):
    import linear_attention_ssm_gated_amd as gdn
    import synth
    d = torch.device("cuda:0")
    K = w.k_rows
    inp = synth.decode_inputs(w.B, K, w.Hk, w.Hv, w.dk, w.dv, seed=w.seed)
    byt = verify_bytes(w.B, w.Hk, w.Hv, w.dk, w.dv, K=K)
    n_sets = max(3, int(ROTATE_BYTES // byt) + 1)
    ssf = gdn.gdn_stash_seq_floats(w.Hv, w.dk, w.dv, K, gdn.GDN_BF16)
    sets = []
    for _ in range(n_sets):
        slots = [inp["states"][b].to(d).clone() for b in range(w.B)]
        sets.append(dict(
            slots=slots,
            table=torch.tensor([s.data_ptr() for s in slots], dtype=torch.int64, device=d),
            q=inp["q"].reshape(w.B * K, -1).to(d), k=inp["k"].reshape(w.B * K, -1).to(d),
            v=inp["v"].reshape(w.B * K, -1).to(d), gate=inp["gate"].reshape(w.B * K, -1).to(d),
            beta=inp["beta"].reshape(w.B * K, -1).to(d),
            out=torch.empty((w.B, K, w.Hv, w.dv), dtype=torch.bfloat16, device=d),
            stash=torch.empty(w.B * ssf, dtype=torch.float32, device=d),
            flag=torch.zeros(1, dtype=torch.int32, device=d)))
    route = []

    def launch(i):   # on the current stream (the capture stream while a graph is recorded)
        g = sets[i]
        r = gdn.gdn_decode_verify_k4(g["table"], g["q"], g["k"], g["v"], g["gate"], g["beta"],
                                     g["out"], g["stash"], w.B, w.Hk, w.Hv, w.dk, w.dv,
                                     w.Hk * w.dk, w.Hv * w.dv, w.Hv, ssf, g["flag"], stream=None)
        if not route:
            route.append(r)

    total_ms, kern_ms, eager_ms, spread = time_launches(launch, n_sets, args.warmup, args.steps, torch)
    ms = total_ms / args.steps
    ach = byt / (kern_ms * 1e-3) / 1e9
    # parity of the timed launches' outputs (the verify writes no state, so every
    # set's outputs are those of the oracle on the same inputs)
    import oracle
    ro, _ = oracle.decode(inp["states"], inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"])
    err = synth.max_rel_err(sets[(args.steps - 1) % n_sets]["out"].float().cpu(), ro)
    # the fold that follows a verify (word set by the verify above), on the same sets
    na_l = inp["na"].tolist()
    for g in sets:
        g["na"] = inp["na"].to(d)

    def launch_fold(i):
        g = sets[i]
        gdn.gdn_fold(g["table"], g["stash"], g["na"], None, 0, g["flag"], K, w.B, w.Hk, w.Hv, w.dk,
                     w.dv, ssf, gdn.GDN_BF16, stream=None)

    _, fold_ms, fold_eager_ms, fold_spread = time_launches(launch_fold, n_sets, args.warmup, args.steps, torch)
    fbyt = fold_bytes(na_l, w.Hv, w.dk, w.dv, K)
    return {
        "metric": "GDN K=4 write-on-accept verify, achieved HBM GB/s (B=16, Hv=48, d=128)",
        "value": ach, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 state, bf16 q/k/v", "data": "synthetic",
        "config": {"workload": w.name, "seed": w.seed, "B": w.B, "K": K, "Hk": w.Hk, "Hv": w.Hv, "dk": w.dk,
                   "dv": w.dv},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(w.name),
                     "algorithmic_bytes": byt, "kernel_ms": kern_ms, "eager_launch_ms": eager_ms, "spread": spread},
        "timing": "median of 11 replays of a HIP graph of the K launches, HIP events around each replay",
        "draft_tokens_per_s": w.B * K / (kern_ms * 1e-3),
        "parity_max_rel_err_out": err,
        "fold": {"kernel_ms": fold_ms, "eager_launch_ms": fold_eager_ms, "spread": fold_spread, "algorithmic_bytes": fbyt, "achieved": fbyt / (fold_ms * 1e-3) / 1e9,
                 "unit": "GB/s", "frac": fbyt / (fold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "na": na_l},
        "route": route[0] if route else None,
        "input_sets_rotated": n_sets,
    }


def bench_step(w, args, torch):
    import linear_attention_ssm_gated_amd as gdn
    import synth
    d = torch.device("cuda:0")
    inp = synth.decode_inputs(w.B, 1, w.Hk, w.Hv, w.dk, w.dv, seed=w.seed)
    byt = step_bytes(w.B, w.Hk, w.Hv, w.dk, w.dv)
    n_sets = max(3, int(ROTATE_BYTES // byt) + 1)
    sets = []
    for _ in range(n_sets):
        slots = [inp["states"][b].to(d).clone() for b in range(w.B)]
        sets.append(dict(
            slots=slots,
            table=torch.tensor([s.data_ptr() for s in slots], dtype=torch.int64, device=d),
            q=inp["q"].reshape(w.B, -1).to(d), k=inp["k"].reshape(w.B, -1).to(d),
            v=inp["v"].reshape(w.B, -1).to(d), gate=inp["gate"].reshape(w.B, -1).to(d),
            beta=inp["beta"].reshape(w.B, -1).to(d),
            out=torch.empty((w.B, w.Hv, w.dv), dtype=torch.bfloat16, device=d)))
    route = []

    def launch(i):   # on the current stream (the capture stream while a graph is recorded)
        g = sets[i]
        r = gdn.gdn_decode_step(g["table"], g["q"], g["k"], g["v"], g["gate"], g["beta"], g["out"],
                                w.B, w.Hk, w.Hv, w.dk, w.dv, w.Hk * w.dk, w.Hv * w.dv, w.Hv,
                                stream=None)
        if not route:
            route.append(r)

    # parity of one step on fresh states (before the timed launches move them on)
    import oracle
    launch(0)
    torch.cuda.synchronize()
    ro, after = oracle.decode(inp["states"], inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"])
    err_out = synth.max_rel_err(sets[0]["out"].float().cpu(), ro[:, 0])
    err_state = max(synth.max_rel_err(sets[0]["slots"][b].cpu(), after[b, 1]) for b in range(w.B))
    total_ms, kern_ms, eager_ms, spread = time_launches(launch, n_sets, args.warmup, args.steps, torch)
    ach = byt / (kern_ms * 1e-3) / 1e9
    return {
        "metric": "GDN K=1 decode step, achieved HBM GB/s (B=16, Hv=48, d=128)",
        "value": ach, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 state, bf16 q/k/v", "data": "synthetic",
        "config": {"workload": w.name, "seed": w.seed, "B": w.B, "K": 1, "Hk": w.Hk, "Hv": w.Hv, "dk": w.dk,
                   "dv": w.dv},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(w.name),
                     "algorithmic_bytes": byt, "kernel_ms": kern_ms, "eager_launch_ms": eager_ms, "spread": spread},
        "timing": "median of 11 replays of a HIP graph of the K launches, HIP events around each replay",
        "tokens_per_s": w.B / (kern_ms * 1e-3),
        "parity_max_rel_err_out": err_out, "parity_max_rel_err_state": err_state,
        "route": route[0] if route else None,
        "input_sets_rotated": n_sets,
    }


def bench_ba(args, torch):
    import linear_attention_ssm_gated_amd as gdn
    import synth
    wl = synth.BA_WORKLOAD
    m, k, nv, G = wl["m"], wl["k"], wl["nv"], wl["vheads_per_group"]
    d = torch.device("cuda:0")
    inp = synth.ba_inputs(m, k, nv, seed=wl["seed"])
    byt = ba_bytes(m, k, nv)
    n_sets = max(3, int(ROTATE_BYTES // byt) + 1)
    ws = torch.empty(gdn.gdn_ba_gates_workspace_bytes(m, 2 * nv, k), dtype=torch.uint8, device=d)
    sets = [dict(x=inp["x"].to(d), w=inp["w"].to(d), a_log=inp["a_log"].to(d), dt_bias=inp["dt_bias"].to(d),
                 out=torch.empty((m, 2 * nv), dtype=torch.float32, device=d)) for _ in range(n_sets)]
    route = []

    def launch(i):   # on the current stream (the capture stream while a graph is recorded)
        g = sets[i]
        r = gdn.gdn_ba_gates(g["x"], g["w"], g["a_log"], g["dt_bias"], g["out"], m, 2 * nv, k, k, 2 * nv,
                             nv, G, workspace=ws, stream=None)
        if not route:
            route.append(r)

    # parity of the first launch on a sample of tokens (fp64 oracle)
    import oracle
    launch(0)
    torch.cuda.synchronize()
    rows = list(range(0, m, 97))
    ref = oracle.ba_gates(inp["x"][rows], inp["w"], inp["a_log"], inp["dt_bias"], nv, G)
    err = synth.max_rel_err(sets[0]["out"][rows].double().cpu().numpy(), ref)
    total_ms, kern_ms, eager_ms, spread = time_launches(launch, n_sets, args.warmup, args.steps, torch)
    ach = byt / (kern_ms * 1e-3) / 1e9
    return {
        "metric": "GDN gate/beta producer (BA projection), achieved HBM GB/s (m=4576, k=5120, n=96)",
        "value": ach, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 x and weight, fp32 accumulation and gates", "data": "synthetic",
        "config": {"workload": wl["name"], "seed": wl["seed"], "m": m, "k": k, "n": 2 * nv, "nv": nv,
                   "vheads_per_group": G},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(wl["name"]),
                     "algorithmic_bytes": byt, "algorithmic_flops": 2.0 * m * k * 2 * nv,
                     "kernel_ms": kern_ms, "eager_launch_ms": eager_ms, "spread": spread},
        "timing": "median of 11 replays of a HIP graph of the K launches, HIP events around each replay",
        "tokens_per_s": m / (kern_ms * 1e-3),
        "parity_max_rel_err_sampled_tokens": err,
        "route": route[0] if route else None,
        "input_sets_rotated": n_sets,
    }


def with_copy_yardstick(rec, torch):
    """Add the measured copy rate and the fraction of it that the path reaches."""
    copy = achievable_copy_gbs(torch)
    r = rec["roofline"]
    r["copy_GBs"] = copy
    r["frac_of_copy"] = r["achieved"] / copy
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="with the default workload, skip the extra verify/fold keys")
    ap.add_argument("--segmented", action="store_true",
                    help="time a prefill workload through gdn_chunk_prefill_segmented (the segment "
                         "scan where it is taken, e.g. --workload prefill_t4576_hv6)")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run plain device-to-device copies of MIB MiB (the known-size "
                         "kernel that scales FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is a design note, not a code path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}), flush=True)
        return
    if args.workload == synth.BA_WORKLOAD["name"]:
        print(json.dumps(with_copy_yardstick(bench_ba(args, torch), torch)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    if w.kind == "prefill":
        rec = bench_prefill(w, args, torch)
        if args.workload == DEFAULT_WORKLOAD and not args.prefill_only:
            # the K = 4 verify and its fold, timed the same way, as extra keys
            v = bench_verify(synth.WORKLOADS["verify_k4_b16"], args, torch)
            rec["decode_verify_k4"] = {
                "workload": v["config"]["workload"], "config": v["config"],
                "roofline": {k: v["roofline"][k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                                          "traffic", "algorithmic_bytes", "kernel_ms", "spread")},
                "draft_tokens_per_s": v["draft_tokens_per_s"], "parity_max_rel_err_out": v["parity_max_rel_err_out"],
                "route": v["route"]}
            f = v["fold"]
            rec["fold_k4"] = {"roofline": {"bound": "hbm", "achieved": f["achieved"], "peak": HBM_PEAK_GBS,
                                           "unit": "GB/s", "frac": f["frac"],
                                           "traffic": measured_kernel_traffic("verify_k4_b16", "fold"),
                                           "algorithmic_bytes": f["algorithmic_bytes"],
                                           "kernel_ms": f["kernel_ms"], "spread": f["spread"]},
                              "na": f["na"]}
            # one GPU's share of the layer (6 v-heads over 2 k-heads): the plain
            # spine and the segment scan, timed the same way
            import types
            nw = synth.WORKLOADS["prefill_t4576_hv6"]
            narrow = {}
            for seg in (False, True):
                a2 = types.SimpleNamespace(**{**vars(args), "no_cpu_baseline": True, "segmented": seg})
                r2 = bench_prefill(nw, a2, torch)
                narrow["segment_scan" if seg else "plain_spine"] = {
                    "ms_per_call": r2["ms_per_step"], "tokens_per_s": r2["value"], "route": r2["route"],
                    "spread": r2["roofline"]["spread"],
                    "parity_max_rel_err_sampled_heads": r2["parity_max_rel_err_sampled_heads"]}
            narrow["speedup"] = narrow["plain_spine"]["ms_per_call"] / narrow["segment_scan"]["ms_per_call"]
            narrow["config"] = {"workload": nw.name, "seed": nw.seed, "B": nw.B, "T": nw.T, "Hk": nw.Hk,
                                "Hv": nw.Hv, "dk": nw.dk, "dv": nw.dv, "chunk": nw.chunk, "h0": nw.h0}
            rec["prefill_hv6"] = narrow
    elif w.kind == "decode_step":
        rec = bench_step(w, args, torch)
    else:
        rec = bench_verify(w, args, torch)
    print(json.dumps(with_copy_yardstick(rec, torch)), flush=True)


if __name__ == "__main__":
    main()
