"""GPU parity and bookkeeping of the parent-mode verify and the fold's restore
branch (ssm_gdn_woa.rs, doc of gdn_wy4_fold: with the engaged word clear the
parent kernel ran, and a partial accept na < k_rows restores Hi(na - 1) from
hi_tables).  The slab reading is the library's (include/gdn.h): slab j of a
sequence is the state after its first j rows, and the parent verify advances
the state itself through all k_rows rows.

Checks, against the fp64 oracle's per-prefix states after[b, j]:
  * outputs of all rows (fp32 <= 1e-4, bf16 within its rounding);
  * the engaged word stays clear;
  * slab 0 is a bitwise copy of the state before the verify, slab j >= 1
    matches after[b, j] (<= 1e-4 of max|state|), slabs past k_rows keep
    their bytes;
  * the state after the verify matches after[b, k_rows];
  * the fold then restores: na < k_rows gives a bitwise copy of slab na,
    na = k_rows keeps the advanced state bitwise; slots outside the table
    keep their bytes;
  * with the word set (a write-on-accept verify ran) the fold ignores the
    slabs and applies the stashed rows.
"""
import numpy as np
import pytest
import torch

import linear_attention_ssm_gated_amd as gdn
import synth
from gpu_common import dev, rel_err, say
from test_gpu_decode import Setup, oracle_decode

pytestmark = pytest.mark.gpu
SENTINEL = -3.5


def make_slabs(s, n_slabs):
    slabs = [torch.full((n_slabs, s.Hv, s.dk, s.dv), SENTINEL, device=dev()) for _ in range(s.B)]
    table = torch.tensor([t.data_ptr() for t in slabs], dtype=torch.int64, device=dev())
    return slabs, table


def parent_verify(s, table, n_slabs):
    return gdn.gdn_decode_verify_parent(s.h_table, table, n_slabs, s.q, s.k, s.v, s.gate, s.beta, s.out,
                                        s.stash, s.B, s.Hk, s.Hv, s.dk, s.dv, s.K, s.qk_stride,
                                        s.v_stride, s.gb_stride, s.ssf)


def fold(s, table, n_slabs):
    return gdn.gdn_fold(s.h_table, s.stash, s.na, table, n_slabs, s.flag, s.K, s.B, s.Hk, s.Hv, s.dk,
                        s.dv, s.ssf, s.io_code)


def check_parent(inp, io, out_dtype, out_tol, route_prefix, slab_pad=1, qk_pad=0):
    s = Setup(inp, io, out_dtype, qk_pad=qk_pad)
    K = s.K
    n_slabs = K + slab_pad
    slabs, table = make_slabs(s, n_slabs)
    before = s.states()
    spares_before = [x.cpu() for x in s.spares]
    s.clear()
    route = parent_verify(s, table, n_slabs)
    torch.cuda.synchronize()
    assert route.startswith(route_prefix), route
    assert int(s.flag.item()) == 0, "the parent verify leaves the engaged word clear"
    ro, after = oracle_decode(inp)
    assert rel_err(s.out, ro) <= out_tol
    advanced = s.states()
    worst = 0.0
    for b in range(s.B):
        sl = slabs[b].cpu()
        assert torch.equal(sl[0], before[b]), f"slab 0 of sequence {b} is the state before the verify"
        for j in range(1, K):
            e = rel_err(sl[j], after[b, j])
            worst = max(worst, e)
            assert e <= 1e-4, (b, j, e)
        assert (sl[K:] == SENTINEL).all(), f"slabs past k_rows of sequence {b} must keep their bytes"
        e = rel_err(advanced[b], after[b, K])
        worst = max(worst, e)
        assert e <= 1e-4, (b, e)
    say("  worst slab/state error", f"{worst:.2e}")
    route = fold(s, table, n_slabs)
    torch.cuda.synchronize()
    assert "gdn_restore_kernel" in route, route
    got = s.states()
    na = np.clip(inp["na"].numpy(), 0, K)
    for b in range(s.B):
        if na[b] < K:
            assert torch.equal(got[b], slabs[b][na[b]].cpu()), f"sequence {b} na={na[b]} restores slab na"
        else:
            assert torch.equal(got[b], advanced[b]), f"sequence {b} na=K keeps the advanced state"
    for x, y in zip(s.spares, spares_before):
        assert torch.equal(x.cpu(), y), "a slot outside the table changed"
    return na


def test_parent_workload_k4():
    """The verify_k4_b16 workload (16 sequences, 48 v-heads, d = 128, bf16)."""
    w = synth.WORKLOADS["verify_k4_b16"]
    inp = synth.decode_inputs(w.B, 4, w.Hk, w.Hv, w.dk, w.dv, io=torch.bfloat16, seed=w.seed)
    say("parent verify_k4_b16")
    na = check_parent(inp, torch.bfloat16, torch.float32, 1e-4, "gdn_verify_d128_kernel+gdn_slab_kernel grid=[48,16,1]")
    assert (na == 0).any() and (na == 4).any() and ((na > 0) & (na < 4)).any(), "every branch exercised"


@pytest.mark.parametrize("K", [1, 3, 8])
def test_parent_rows_d128(K):
    inp = synth.decode_inputs(6, K, 2, 6, 128, 128, io=torch.bfloat16, seed=700 + K)
    inp["na"] = torch.arange(6, dtype=torch.int32) % (K + 1)   # 0 .. K, and K again
    say("parent rows d128", K)
    check_parent(inp, torch.bfloat16, torch.bfloat16, 4e-3, f"gdn_verify_d128_kernel+gdn_slab_kernel grid=[6,6,1]",
                 slab_pad=2, qk_pad=8)


@pytest.mark.parametrize("K,io", [(2, torch.float32), (5, torch.bfloat16)])
def test_parent_generic(K, io):
    inp = synth.decode_inputs(5, K, 1, 3, 64, 96, io=io, seed=720 + K)
    inp["na"] = torch.tensor([0, K, 1, K - 1, 7], dtype=torch.int32)   # 7 clamps to K
    say("parent generic", K, io)
    check_parent(inp, io, torch.float32, 1e-4, "gdn_verify_kernel+gdn_slab_kernel grid=[3,5,1]")


def test_restore_not_taken_when_the_word_is_set():
    """A write-on-accept verify ran (word set): the fold applies the stashed
    rows, and the slab table passed alongside is not read."""
    inp = synth.decode_inputs(4, 4, 2, 6, 128, 128, io=torch.bfloat16, seed=741)
    inp["na"] = torch.tensor([0, 4, 2, 1], dtype=torch.int32)
    s = Setup(inp, torch.bfloat16, torch.float32)
    slabs, table = make_slabs(s, 4)
    before = s.states()
    s.clear()
    s.verify()
    torch.cuda.synchronize()
    assert int(s.flag.item()) == 1
    fold(s, table, 4)
    torch.cuda.synchronize()
    _, after = oracle_decode(inp)
    got = s.states()
    for b in range(s.B):
        na = int(inp["na"][b])
        if na == 0:
            assert torch.equal(got[b], before[b])
        else:
            assert rel_err(got[b], after[b, na]) <= 1e-4, (b, na)
        assert (slabs[b].cpu() == SENTINEL).all(), "the slabs were not written"
