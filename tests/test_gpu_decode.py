"""GPU parity and bookkeeping of the write-on-accept verify (K = 4, and any K in
1..8), its fold, and the in-place K = 1 decode step.

States sit in separately allocated slots, allocated in shuffled order and
interleaved with spare slots that are not in the pointer table.  Checks:
  * outputs of all 4 rows against the fp64 oracle (fp32 outputs <= 1e-4,
    bf16 outputs within bf16 rounding, 4e-3);
  * verify writes no state (bitwise) and sets the engaged word;
  * after the fold, each state equals the oracle's state after its first na
    rows (<= 1e-4 of max|state|); na = 0 states and spare slots are bitwise
    unchanged;
  * one-hot keys with no decay and beta = 1 make the accepted rows
    identifiable: exactly rows 0..na-1 of each state change, bit for bit;
  * with the word cleared (no verify since the clear) the fold changes nothing;
  * repeated runs are bitwise identical;
  * K = 1..8 on both kernel paths: outputs and folded states against the
    oracle, the stash padding untouched;
  * the K = 1 step: outputs and updated states against the oracle, slots
    outside the table untouched, and two steps in a row equal the oracle's
    two-row chunk.
"""
import numpy as np
import pytest
import torch

import linear_attention_ssm_gated_amd as gdn
import oracle
import synth
from gpu_common import dev, rel_err, say

pytestmark = pytest.mark.gpu
K = 4


class Setup:
    def __init__(self, inp, io, out_dtype, qk_pad=0, stash_pad=0):
        d = dev()
        st = inp["states"]
        self.B, self.Hv, self.dk, self.dv = st.shape
        self.Hk = inp["q"].shape[2]
        self.K = K = inp["q"].shape[1]
        B, Hv, dk, dv, Hk = self.B, self.Hv, self.dk, self.dv, self.Hk
        self.io = io
        # separately allocated states, in shuffled order, with spare slots between
        self.slots = [None] * B
        self.spares = []
        for idx in inp["slot_perm"].tolist():
            self.spares.append(torch.full((Hv, dk, dv), -7.25, device=d))
            self.slots[idx] = st[idx].to(d).clone()
        self.h_table = torch.tensor([s.data_ptr() for s in self.slots], dtype=torch.int64, device=d)
        # rows with padded strides
        self.qk_stride = Hk * dk + qk_pad
        self.v_stride = Hv * dv + qk_pad
        self.gb_stride = Hv + qk_pad

        def rows(x, width, stride, dtype):
            buf = torch.zeros((B * K, stride), dtype=dtype)
            buf[:, :width] = x.reshape(B * K, width).to(dtype)
            return buf.to(d)

        self.q = rows(inp["q"], Hk * dk, self.qk_stride, io)
        self.k = rows(inp["k"], Hk * dk, self.qk_stride, io)
        self.v = rows(inp["v"], Hv * dv, self.v_stride, io)
        self.gate = rows(inp["gate"], Hv, self.gb_stride, torch.float32)
        self.beta = rows(inp["beta"], Hv, self.gb_stride, torch.float32)
        self.out = torch.empty((B, K, Hv, dv), dtype=out_dtype, device=d)
        self.io_code = gdn.GDN_BF16 if io == torch.bfloat16 else gdn.GDN_F32
        self.ssf = gdn.gdn_stash_seq_floats(Hv, dk, dv, K, self.io_code) + stash_pad
        self.stash_pad = stash_pad
        self.stash = torch.full((B * self.ssf,), float("nan"), device=d)
        self.flag = torch.full((1,), 7, dtype=torch.int32, device=d)
        self.na = inp["na"].to(d)

    def states(self):
        return torch.stack([s for s in self.slots]).cpu()

    def clear(self):
        gdn.gdn_flag_clear(self.flag)

    def verify(self):
        if self.K == 4:   # the pages' entry point
            return gdn.gdn_decode_verify_k4(self.h_table, self.q, self.k, self.v, self.gate, self.beta,
                                            self.out, self.stash, self.B, self.Hk, self.Hv, self.dk,
                                            self.dv, self.qk_stride, self.v_stride, self.gb_stride,
                                            self.ssf, self.flag)
        return gdn.gdn_decode_verify(self.h_table, self.q, self.k, self.v, self.gate, self.beta,
                                     self.out, self.stash, self.B, self.Hk, self.Hv, self.dk, self.dv,
                                     self.K, self.qk_stride, self.v_stride, self.gb_stride, self.ssf,
                                     self.flag)

    def fold(self):
        return gdn.gdn_fold(self.h_table, self.stash, self.na, None, 0, self.flag, self.K, self.B,
                            self.Hk, self.Hv, self.dk, self.dv, self.ssf, self.io_code)

    def step(self):
        """The K = 1 step on row 0 of each sequence (the rows are K = 1 rows)."""
        assert self.K == 1
        return gdn.gdn_decode_step(self.h_table, self.q, self.k, self.v, self.gate, self.beta,
                                   self.out, self.B, self.Hk, self.Hv, self.dk, self.dv,
                                   self.qk_stride, self.v_stride, self.gb_stride)


def oracle_decode(inp):
    return oracle.decode(inp["states"], inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"])


@pytest.mark.parametrize("io,out_dtype,tol,pad", [
    (torch.bfloat16, torch.float32, 1e-4, 0),
    (torch.bfloat16, torch.bfloat16, 4e-3, 0),
    (torch.float32, torch.float32, 1e-4, 0),
    (torch.bfloat16, torch.float32, 1e-4, 24),
])
def test_verify_fold_workload(io, out_dtype, tol, pad):
    w = synth.WORKLOADS["verify_k4_b16"]
    inp = synth.decode_inputs(w.B, K, w.Hk, w.Hv, w.dk, w.dv, io=io, seed=w.seed)
    say("verify_k4_b16", io, out_dtype, "pad", pad)
    s = Setup(inp, io, out_dtype, qk_pad=pad, stash_pad=pad)
    before = s.states()
    spares_before = [x.cpu() for x in s.spares]
    s.clear()
    torch.cuda.synchronize()
    assert int(s.flag.item()) == 0
    route = s.verify()
    torch.cuda.synchronize()
    assert route.startswith("gdn_verify_d128_kernel grid=[48,16,1]"), route
    assert int(s.flag.item()) == 1, "verify marks the engaged word"
    assert torch.equal(s.states(), before), "verify writes no state"
    ro, after = oracle_decode(inp)
    eo = rel_err(s.out, ro)
    assert eo <= tol
    s.fold()
    torch.cuda.synchronize()
    got = s.states()
    na = inp["na"].numpy()
    eh = 0.0
    for b in range(s.B):
        if na[b] == 0:
            assert torch.equal(got[b], before[b]), f"na=0 state {b} must keep its bytes"
        else:
            e = rel_err(got[b], after[b, na[b]])
            eh = max(eh, e)
            assert e <= 1e-4, f"sequence {b} na={na[b]}"
    say(f"  out err {eo:.3e}  folded state err {eh:.3e}")
    for x, y in zip(s.spares, spares_before):
        assert torch.equal(x.cpu(), y), "a slot outside the table changed"


@pytest.mark.parametrize("B,Hk,Hv", [(3, 2, 6), (87, 1, 3), (13, 1, 5)])
def test_d128_shapes_and_stash_bounds(B, Hk, Hv):
    """dk = dv = 128 verify at several batch and head counts, with padded
    rows and a padded stash whose padding must stay untouched."""
    inp = synth.decode_inputs(B, K, Hk, Hv, 128, 128, io=torch.bfloat16, seed=60 + B)
    say("decode d128 shapes", B, Hk, Hv)
    s = Setup(inp, torch.bfloat16, torch.float32, qk_pad=8, stash_pad=16)
    before = s.states()
    s.clear()
    route = s.verify()
    torch.cuda.synchronize()
    assert route.startswith(f"gdn_verify_d128_kernel grid=[{Hv},{B},1]"), route
    stash = s.stash.view(B, s.ssf).cpu()
    assert torch.isnan(stash[:, s.ssf - 16:]).all(), "the stash padding must stay untouched"
    ro, after = oracle_decode(inp)
    assert rel_err(s.out, ro) <= 1e-4
    s.fold()
    torch.cuda.synchronize()
    got = s.states()
    for b in range(B):
        na = int(inp["na"][b])
        if na == 0:
            assert torch.equal(got[b], before[b])
        else:
            assert rel_err(got[b], after[b, na]) <= 1e-4, (b, na)


@pytest.mark.parametrize("dk,dv", [(64, 96), (128, 64), (32, 128)])
def test_generic_shapes(dk, dv):
    """Head sizes other than 128 take the generic verify/fold kernels."""
    inp = synth.decode_inputs(6, K, 2, 4, dk, dv, io=torch.bfloat16, seed=40 + dk + dv)
    say("decode generic", dk, dv)
    s = Setup(inp, torch.bfloat16, torch.float32, qk_pad=8)
    before = s.states()
    s.clear()
    route = s.verify()
    assert route.startswith("gdn_verify_kernel "), route
    s.fold()
    torch.cuda.synchronize()
    ro, after = oracle_decode(inp)
    assert rel_err(s.out, ro) <= 1e-4
    got = s.states()
    for b in range(s.B):
        na = int(inp["na"][b])
        if na == 0:
            assert torch.equal(got[b], before[b])
        else:
            assert rel_err(got[b], after[b, na]) <= 1e-4


def test_fold_without_verify_is_a_no_op():
    inp = synth.decode_inputs(4, K, 2, 4, 128, 128, seed=21)
    say("fold with the word clear")
    s = Setup(inp, torch.bfloat16, torch.float32)
    s.na.fill_(4)
    s.stash.fill_(1.0)
    before = s.states()
    s.clear()
    s.fold()
    torch.cuda.synchronize()
    assert torch.equal(s.states(), before)


def test_one_hot_rows_bookkeeping():
    """gate = 0, beta = 1, key s = e_s: the fold of na rows moves exactly state
    rows 0..na-1 (the others are multiplied by exp(0) = 1 and get 0 * delta)."""
    B, Hk, Hv, dk, dv = 5, 1, 2, 128, 128
    inp = synth.decode_inputs(B, K, Hk, Hv, dk, dv, seed=22)
    k = torch.zeros(B, K, Hk, dk)
    for s_ in range(K):
        k[:, s_, :, s_] = 1.0
    inp["k"] = k.to(torch.bfloat16)
    inp["gate"] = torch.zeros(B, K, Hv)
    inp["beta"] = torch.ones(B, K, Hv)
    inp["v"] = (inp["v"].float() + 3.0).to(torch.bfloat16)  # make every delta nonzero
    say("one-hot bookkeeping")
    s = Setup(inp, torch.bfloat16, torch.float32)
    before = s.states()
    s.clear()
    s.verify()
    s.fold()
    torch.cuda.synchronize()
    got = s.states()
    for b in range(B):
        na = int(inp["na"][b])
        changed = (got[b] != before[b]).any(dim=-1)  # [Hv, dk]
        for vh in range(Hv):
            rows = torch.nonzero(changed[vh]).flatten().tolist()
            assert rows == list(range(na)), (b, vh, na, rows)


def test_verify_fold_deterministic():
    w = synth.WORKLOADS["verify_k4_b16"]
    inp = synth.decode_inputs(w.B, K, w.Hk, w.Hv, w.dk, w.dv, seed=w.seed)
    say("decode determinism")
    res = []
    for _ in range(2):
        s = Setup(inp, torch.bfloat16, torch.bfloat16)
        s.clear()
        s.verify()
        s.fold()
        torch.cuda.synchronize()
        res.append((s.out.cpu(), s.stash.cpu(), s.states()))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def check_verify_fold(inp, s, route_prefix, out_tol):
    B = s.B
    before = s.states()
    spares_before = [x.cpu() for x in s.spares]
    s.clear()
    route = s.verify()
    torch.cuda.synchronize()
    assert route.startswith(route_prefix), route
    assert int(s.flag.item()) == 1
    assert torch.equal(s.states(), before), "verify writes no state"
    if s.stash_pad:
        pad = s.stash.view(B, s.ssf).cpu()[:, s.ssf - s.stash_pad:]
        assert torch.isnan(pad).all(), "the stash padding must stay untouched"
    ro, after = oracle_decode(inp)
    assert rel_err(s.out, ro) <= out_tol
    s.fold()
    torch.cuda.synchronize()
    got = s.states()
    for b in range(B):
        na = int(inp["na"][b])
        if na == 0:
            assert torch.equal(got[b], before[b]), b
        else:
            assert rel_err(got[b], after[b, na]) <= 1e-4, (b, na)
    for x, y in zip(s.spares, spares_before):
        assert torch.equal(x.cpu(), y)


@pytest.mark.parametrize("K", [1, 2, 3, 5, 8])
def test_verify_fold_any_rows_d128(K):
    inp = synth.decode_inputs(6, K, 2, 6, 128, 128, io=torch.bfloat16, seed=300 + K)
    say("verify rows d128", K)
    s = Setup(inp, torch.bfloat16, torch.float32, qk_pad=8, stash_pad=16)
    check_verify_fold(inp, s, "gdn_verify_d128_kernel grid=[6,6,1]", 1e-4)


@pytest.mark.parametrize("K,io", [(1, torch.float32), (3, torch.bfloat16), (8, torch.float32)])
def test_verify_fold_any_rows_generic(K, io):
    inp = synth.decode_inputs(5, K, 1, 3, 64, 96, io=io, seed=320 + K)
    say("verify rows generic", K, io)
    s = Setup(inp, io, torch.float32, qk_pad=4, stash_pad=8)
    check_verify_fold(inp, s, "gdn_verify_kernel grid=[3,5,1]", 1e-4)


def test_verify_rows8_d128_bf16_out():
    inp = synth.decode_inputs(16, 8, 16, 48, 128, 128, io=torch.bfloat16, seed=341)
    say("verify rows d128 K=8 full heads")
    s = Setup(inp, torch.bfloat16, torch.bfloat16)
    check_verify_fold(inp, s, "gdn_verify_d128_kernel grid=[48,16,1]", 4e-3)


def check_step(inp, s, route_prefix, out_tol):
    spares_before = [x.cpu() for x in s.spares]
    route = s.step()
    torch.cuda.synchronize()
    assert route.startswith(route_prefix), route
    ro, after = oracle_decode(inp)
    assert rel_err(s.out[:, 0], ro[:, 0]) <= out_tol
    got = s.states()
    for b in range(s.B):
        assert rel_err(got[b], after[b, 1]) <= 1e-4, b
    for x, y in zip(s.spares, spares_before):
        assert torch.equal(x.cpu(), y), "a slot outside the table changed"


@pytest.mark.parametrize("io,out_dtype,tol", [
    (torch.bfloat16, torch.float32, 1e-4),
    (torch.bfloat16, torch.bfloat16, 4e-3),
    (torch.float32, torch.float32, 1e-4),
])
def test_step_d128(io, out_dtype, tol):
    inp = synth.decode_inputs(16, 1, 16, 48, 128, 128, io=io, seed=360)
    say("step d128", io, out_dtype)
    s = Setup(inp, io, out_dtype, qk_pad=8)
    check_step(inp, s, "gdn_step_d128_kernel grid=[48,16,1]", tol)


@pytest.mark.parametrize("dk,dv", [(64, 96), (128, 64), (33, 128)])
def test_step_generic(dk, dv):
    inp = synth.decode_inputs(5, 1, 2, 4, dk, dv, io=torch.bfloat16, seed=370 + dk + dv)
    say("step generic", dk, dv)
    s = Setup(inp, torch.bfloat16, torch.float32, qk_pad=2)
    check_step(inp, s, "gdn_step_kernel grid=[4,5,1]", 1e-4)


@pytest.mark.parametrize("dk", [128, 64])
def test_two_steps_equal_the_two_row_chunk(dk):
    """Two K = 1 steps on rows 0 and 1 give the oracle's outputs and state
    after both rows of the same two-row chunk."""
    inp2 = synth.decode_inputs(4, 2, 1, 3, dk, dk, io=torch.bfloat16, seed=380 + dk)
    say("two steps", dk)
    ro, after = oracle_decode(inp2)
    rows = []
    for r in range(2):
        inp1 = dict(inp2)
        for name in ("q", "k", "v", "gate", "beta"):
            inp1[name] = inp2[name][:, r:r + 1]
        rows.append(inp1)
    s = Setup(rows[0], torch.bfloat16, torch.float32)
    s.step()
    out0 = s.out.clone()
    s1 = Setup(rows[1], torch.bfloat16, torch.float32)
    # the second step runs on the states the first one left
    s1.slots, s1.h_table = s.slots, s.h_table
    s1.step()
    torch.cuda.synchronize()
    assert rel_err(out0[:, 0], ro[:, 0]) <= 1e-4
    assert rel_err(s1.out[:, 0], ro[:, 1]) <= 1e-4
    got = torch.stack([x for x in s.slots]).cpu()
    for b in range(4):
        assert rel_err(got[b], after[b, 2]) <= 1e-4, b
