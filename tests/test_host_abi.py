"""Host-side checks of the C ABI, no GPU needed.

The library must load, export every entry point include/gdn.h declares, and
refuse each bad argument with its own named status before launching anything
(the *_plan entry points run the same validation as the launching ones and
stop there).  Pointers below are dummies: the plan functions only compare them
with NULL.
"""
import os
import re

import pytest

import linear_attention_ssm_gated_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
X = 0x1000  # non-NULL dummy pointer


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn.so is not built (run __graft_entry__.build())")
    return gdn.library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 23, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gdn.h but not exported"
    assert set(names) == set(gdn.SIGNATURES), "binding and header disagree"


def test_status_strings_are_distinct(lib):
    texts = [gdn.status_string(s) for s in range(12)]
    assert len(set(texts)) == 12
    for s, t in enumerate(texts):
        assert t.startswith(gdn._STATUS[s]), (s, t)
    assert gdn.status_string(99) == "unknown gdn status"


def prefill_plan(lib, **kw):
    a = dict(q=X, k=X, v=X, log_g=X, beta=X, h0=None, out=X, h_final=X, B=1, T=128, Hk=16, Hv=48,
             dk=128, dv=128, chunk=64, cu=None, io=1, od=1, ws=X, ws_bytes=1 << 40)
    a.update(kw)
    return lib.gdn_chunk_prefill_plan(a["q"], a["k"], a["v"], a["log_g"], a["beta"], a["h0"],
                                      a["out"], a["h_final"], a["B"], a["T"], a["Hk"], a["Hv"],
                                      a["dk"], a["dv"], a["chunk"], a["cu"], a["io"], a["od"],
                                      a["ws"], a["ws_bytes"])


def test_prefill_routes(lib):
    assert prefill_plan(lib) == 0
    r = gdn.last_route()
    assert r.startswith("gdn_wy_prep_kernel+gdn_spine_kernel grid=[192,1,1] block=256"), r
    assert "lds=" in r
    # fp32 I/O goes to the generic kernel and the line says why
    assert prefill_plan(lib, io=0, od=0, dk=32, dv=32, chunk=32, Hk=1, Hv=1) == 0
    r = gdn.last_route()
    assert r.startswith("gdn_prefill_generic_kernel") and "io dtype is f32" in r, r
    assert "grid=[1,1,1]" in r
    # bf16 with an odd head size: generic, naming the dk/dv guard
    assert prefill_plan(lib, dk=64, dv=96) == 0
    r = gdn.last_route()
    assert r.startswith("gdn_prefill_generic_kernel") and "dk = dv = 128" in r, r
    assert "grid=[144,1,1]" in r  # 48 v-heads x 3 column slices of 32
    assert prefill_plan(lib, chunk=32) == 0
    assert "chunk = 64" in gdn.last_route()


def segmented_plan(lib, **kw):
    a = dict(q=X, k=X, v=X, log_g=X, beta=X, h0=None, out=X, h_final=X, B=1, T=4576, Hk=2, Hv=6,
             dk=128, dv=128, chunk=64, cu=None, io=1, od=1, ws=X, ws_bytes=1 << 40)
    a.update(kw)
    return lib.gdn_chunk_prefill_segmented_plan(a["q"], a["k"], a["v"], a["log_g"], a["beta"], a["h0"],
                                                a["out"], a["h_final"], a["B"], a["T"], a["Hk"], a["Hv"],
                                                a["dk"], a["dv"], a["chunk"], a["cu"], a["io"], a["od"],
                                                a["ws"], a["ws_bytes"])


SEG_ROUTE = ("gdn_wy_prep_kernel+gdn_spine_kernel(segment maps)+gdn_segment_combine_kernel"
             "+gdn_spine_kernel(segment outputs)")


@pytest.mark.parametrize("B,T,Hv,S", [
    (1, 4576, 6, 6),      # 24 spine workgroups: (256 // 24 + 3) // 2 = 6 segments of 12 chunks
    (2, 2373, 3, 6),      # 38 chunks: 6 segments of 7 chunks, the last one of 3
    (1, 2560, 2, 10),     # capped at 10 segments (the combine's 8 unrolled steps)
    (1, 192, 1, 3),       # 3 chunks: 3 one-chunk segments
    (1, 577, 6, 5),       # 10 chunks, the last holding one row: 5 segments of 2
])
def test_segment_cut(lib, B, T, Hv, S):
    assert segmented_plan(lib, B=B, T=T, Hk=1, Hv=Hv) == 0
    r = gdn.last_route()
    assert r.startswith(f"{SEG_ROUTE} grid=[{Hv * 4},{B * S},1]"), r


def test_segmented_falls_back(lib):
    # packed input, a spine that fills more than a third of the chip, and too
    # few chunks for three segments: the plain spine, and the line says why
    assert segmented_plan(lib, B=2, T=1000, cu=X) == 0
    r = gdn.last_route()
    assert r.startswith("gdn_wy_prep_kernel+gdn_spine_kernel grid=[24,2,1]") and "dense input" in r, r
    assert segmented_plan(lib, Hk=4, Hv=24, T=700) == 0
    r = gdn.last_route()
    assert r.startswith("gdn_wy_prep_kernel+gdn_spine_kernel grid=[96,1,1]") and "fill the chip" in r, r
    assert segmented_plan(lib, T=128) == 0
    assert gdn.last_route().startswith("gdn_wy_prep_kernel+gdn_spine_kernel grid=[24,1,1]")
    # other shapes run the generic kernel, as gdn_chunk_prefill would
    assert segmented_plan(lib, dk=64, dv=64) == 0
    assert gdn.last_route().startswith("gdn_prefill_generic_kernel")


def test_segmented_workspace(lib):
    # the public size covers the segment scan: the slots, then 3 fp32 128 x 128
    # matrices per (segment, v-head); the plain route asks only its own size
    plain = 256 + 72 * 6 * 2 * 7168
    full = gdn.gdn_prefill_workspace_bytes(1, 4576, 2, 6, 128, 128, 64, 1)
    assert full == 72 * 6 * 2 * 7168 + 3 * 6 * 6 * 128 * 128 * 4
    assert segmented_plan(lib, ws_bytes=full) == 0
    assert segmented_plan(lib, ws_bytes=full - 1) == 6
    assert prefill_plan(lib, T=4576, Hk=2, Hv=6, ws_bytes=plain) == 0
    assert prefill_plan(lib, T=4576, Hk=2, Hv=6, ws_bytes=plain - 1) == 6
    # where the cut is not taken, both routes ask the same
    assert gdn.gdn_prefill_workspace_bytes(1, 4576, 16, 48, 128, 128, 64, 1) == 256 + 72 * 48 * 2 * 7168


@pytest.mark.parametrize("kw,status", [
    (dict(io=2), 5), (dict(od=-1), 5),
    (dict(B=0), 2), (dict(T=-1), 2), (dict(Hk=0), 2), (dict(dk=0), 2), (dict(chunk=0), 2),
    (dict(B=70000), 2),
    (dict(Hk=5), 3),
    (dict(dk=129), 4), (dict(dv=256), 4), (dict(chunk=65), 4),
    (dict(q=None), 1), (dict(out=None), 1), (dict(beta=None), 1),
    (dict(ws=None), 6), (dict(ws_bytes=1000), 6), (dict(Hv=70000, Hk=70000), 2),
])
def test_prefill_refusals(lib, kw, status):
    assert prefill_plan(lib, **kw) == status
    r = gdn.last_route()
    assert "refused" in r and gdn._STATUS[status] in r, r


def test_prefill_empty_needs_no_pointers(lib):
    assert prefill_plan(lib, T=0, q=None, k=None, v=None, log_g=None, beta=None, out=None) == 0


def test_workspace_and_stash_sizes(lib):
    # MFMA route: a 256-byte chunk table, then per (chunk, v-head) T diag(beta) and P,
    # each 64 x 64 bf16 (6 KiB) plus the chunk's per-row decay factors (1 KiB)
    assert gdn.gdn_prefill_workspace_bytes(1, 4576, 16, 48, 128, 128, 64, 1) == 256 + 72 * 48 * 2 * 7168
    assert gdn.gdn_prefill_workspace_bytes(2, 100, 16, 48, 128, 128, 64, 1) == 256 + 2 * 2 * 48 * 2 * 7168
    # packed: ceil(T / 64) + B chunks at most
    assert gdn.gdn_prefill_workspace_bytes(8, 39168, 16, 48, 128, 128, 64, 1, packed=True) == \
        256 + (612 + 8) * 48 * 2 * 7168
    # generic route needs none
    assert gdn.gdn_prefill_workspace_bytes(1, 4576, 16, 48, 128, 128, 64, 0) == 0
    assert gdn.gdn_prefill_workspace_bytes(1, 4576, 16, 48, 64, 64, 64, 1) == 0
    # per v-head: delta K*dv, G K, keys K*dk bf16 (ceil(K*dk/2) floats) or fp32 (K*dk floats)
    assert gdn.gdn_stash_seq_floats(48, 128, 128, 4, 1) == 48 * (4 * 128 + 4 + 2 * 128)
    assert gdn.gdn_stash_seq_floats(48, 128, 128, 4, 0) == 48 * (4 * 128 + 4 + 4 * 128)
    assert gdn.gdn_stash_seq_floats(48, 128, 128, 3, 1) == 48 * (3 * 128 + 3 + 192)
    assert gdn.gdn_stash_seq_floats(2, 33, 64, 1, 1) == 2 * (64 + 1 + 17)
    assert gdn.gdn_stash_seq_floats(2, 33, 64, 8, 0) == 2 * (8 * 64 + 8 + 8 * 33)
    assert gdn.gdn_stash_seq_floats(48, 128, 128, 0, 1) == 0
    assert gdn.gdn_stash_seq_floats(48, 128, 128, 9, 1) == 0


def verify_plan(lib, **kw):
    a = dict(ht=X, q=X, k=X, v=X, gate=X, beta=X, out=X, stash=X, B=16, Hk=16, Hv=48, dk=128,
             dv=128, qks=16 * 128, vs=48 * 128, gbs=48, ssf=48 * (512 + 4 + 256), flag=X, io=1, od=1)
    a.update(kw)
    return lib.gdn_decode_verify_k4_plan(a["ht"], a["q"], a["k"], a["v"], a["gate"], a["beta"],
                                         a["out"], a["stash"], a["B"], a["Hk"], a["Hv"], a["dk"],
                                         a["dv"], a["qks"], a["vs"], a["gbs"], a["ssf"], a["flag"],
                                         a["io"], a["od"])


def test_verify_plan(lib):
    assert verify_plan(lib) == 0
    r = gdn.last_route()
    assert r.startswith("gdn_verify_d128_kernel grid=[48,16,1] block=256 lds=32416B"), r
    assert verify_plan(lib, dk=64, dv=64, qks=16 * 64, vs=48 * 64, ssf=48 * (256 + 4 + 128)) == 0
    assert gdn.last_route().startswith("gdn_verify_kernel grid=[48,16,1]")


def verify_rows_plan(lib, k_rows, **kw):
    a = dict(ht=X, q=X, k=X, v=X, gate=X, beta=X, out=X, stash=X, B=16, Hk=16, Hv=48, dk=128,
             dv=128, qks=16 * 128, vs=48 * 128, gbs=48, flag=X, io=1, od=1)
    a.update(kw)
    ssf = a.pop("ssf", gdn.gdn_stash_seq_floats(a["Hv"], a["dk"], a["dv"], max(1, min(k_rows, 8)), a["io"]))
    return lib.gdn_decode_verify_plan(a["ht"], a["q"], a["k"], a["v"], a["gate"], a["beta"], a["out"],
                                      a["stash"], a["B"], a["Hk"], a["Hv"], a["dk"], a["dv"], k_rows,
                                      a["qks"], a["vs"], a["gbs"], ssf, a["flag"], a["io"], a["od"])


@pytest.mark.parametrize("k_rows", [1, 2, 3, 5, 8])
def test_verify_any_rows_plan(lib, k_rows):
    assert verify_rows_plan(lib, k_rows) == 0
    assert gdn.last_route().startswith("gdn_verify_d128_kernel grid=[48,16,1] block=256")
    assert verify_rows_plan(lib, k_rows, dk=64, dv=96, qks=16 * 64, vs=48 * 96) == 0
    assert gdn.last_route().startswith("gdn_verify_kernel grid=[48,16,1]")
    # a stash sized for fewer rows is refused
    if k_rows > 1:
        small = gdn.gdn_stash_seq_floats(48, 128, 128, k_rows - 1, 1)
        assert verify_rows_plan(lib, k_rows, ssf=small) == 7


@pytest.mark.parametrize("k_rows", [0, 9, -1])
def test_verify_rows_refused(lib, k_rows):
    assert verify_rows_plan(lib, k_rows, ssf=1 << 20) == 8
    assert "k_rows must be 1..8" in gdn.last_route()


@pytest.mark.parametrize("kw,status", [
    (dict(ht=None), 1), (dict(stash=None), 1), (dict(flag=None), 1), (dict(q=None), 1),
    (dict(B=0), 2), (dict(Hk=7), 3), (dict(dv=130), 4), (dict(dv=126), 4),
    (dict(qks=100), 9), (dict(vs=48 * 128 - 1), 9), (dict(gbs=47), 9),
    (dict(ssf=100), 7), (dict(io=3), 5),
])
def test_verify_refusals(lib, kw, status):
    assert verify_plan(lib, **kw) == status
    assert "refused" in gdn.last_route()


def fold_plan(lib, **kw):
    a = dict(ht=X, stash=X, na=X, hi=None, slab=0, flag=X, k_rows=4, B=16, Hk=16, Hv=48, dk=128,
             dv=128, ssf=48 * (512 + 4 + 256), io=1)
    a.update(kw)
    return lib.gdn_fold_plan(a["ht"], a["stash"], a["na"], a["hi"], a["slab"], a["flag"],
                             a["k_rows"], a["B"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["ssf"], a["io"])


def test_fold_plan(lib):
    assert fold_plan(lib) == 0
    assert gdn.last_route().startswith("gdn_fold_d128_kernel grid=[48,16,4] block=256")
    for k_rows in (1, 3, 8):
        ssf = gdn.gdn_stash_seq_floats(48, 128, 128, k_rows, 1)
        assert fold_plan(lib, k_rows=k_rows, ssf=ssf) == 0
    assert fold_plan(lib, dk=64, dv=64, ssf=48 * (256 + 4 + 128)) == 0
    assert gdn.last_route().startswith("gdn_fold_kernel grid=[48,16,1]")
    # the restore branch: slabs 0 .. k_rows - 1 must exist
    assert fold_plan(lib, hi=X, slab=4) == 0
    assert "gdn_restore_kernel" in gdn.last_route()
    assert fold_plan(lib, hi=X, slab=9) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(k_rows=0), 8), (dict(k_rows=9), 8), (dict(k_rows=5), 7), (dict(hi=X), 10), (dict(hi=X, slab=3), 10),
    (dict(na=None), 1), (dict(ht=None), 1),
    (dict(ssf=10), 7), (dict(Hv=47), 3), (dict(io=9), 5),
])
def test_fold_refusals(lib, kw, status):
    assert fold_plan(lib, **kw) == status
    assert "refused" in gdn.last_route()


def parent_plan(lib, **kw):
    a = dict(ht=X, hi=X, slab=4, q=X, k=X, v=X, gate=X, beta=X, out=X, stash=X, B=16, Hk=16, Hv=48,
             dk=128, dv=128, k_rows=4, qks=16 * 128, vs=48 * 128, gbs=48, ssf=48 * (512 + 4 + 256),
             io=1, od=1)
    a.update(kw)
    return lib.gdn_decode_verify_parent_plan(a["ht"], a["hi"], a["slab"], a["q"], a["k"], a["v"],
                                             a["gate"], a["beta"], a["out"], a["stash"], a["B"], a["Hk"],
                                             a["Hv"], a["dk"], a["dv"], a["k_rows"], a["qks"], a["vs"],
                                             a["gbs"], a["ssf"], a["io"], a["od"])


def test_parent_verify_plan(lib):
    assert parent_plan(lib) == 0
    assert gdn.last_route().startswith("gdn_verify_d128_kernel+gdn_slab_kernel grid=[48,16,1] block=256")
    assert parent_plan(lib, dk=64, dv=64, qks=16 * 64, vs=48 * 64, ssf=48 * (256 + 4 + 128)) == 0
    assert gdn.last_route().startswith("gdn_verify_kernel+gdn_slab_kernel grid=[48,16,1]")


@pytest.mark.parametrize("kw,status", [
    (dict(hi=None), 1), (dict(ht=None), 1), (dict(stash=None), 1), (dict(slab=3), 10), (dict(slab=0), 10),
    (dict(k_rows=9), 8), (dict(ssf=10), 7), (dict(Hv=47), 3), (dict(io=9), 5), (dict(qks=100), 9),
])
def test_parent_verify_refusals(lib, kw, status):
    assert parent_plan(lib, **kw) == status
    assert "refused" in gdn.last_route()


def step_plan(lib, **kw):
    a = dict(ht=X, q=X, k=X, v=X, gate=X, beta=X, out=X, B=16, Hk=16, Hv=48, dk=128, dv=128,
             qks=16 * 128, vs=48 * 128, gbs=48, io=1, od=1)
    a.update(kw)
    return lib.gdn_decode_step_plan(a["ht"], a["q"], a["k"], a["v"], a["gate"], a["beta"], a["out"],
                                    a["B"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["qks"], a["vs"],
                                    a["gbs"], a["io"], a["od"])


def test_step_plan(lib):
    assert step_plan(lib) == 0
    assert gdn.last_route().startswith("gdn_step_d128_kernel grid=[48,16,1] block=256")
    assert step_plan(lib, dk=32, dv=96, qks=16 * 32, vs=48 * 96) == 0
    assert gdn.last_route().startswith("gdn_step_kernel grid=[48,16,1] block=256")


@pytest.mark.parametrize("kw,status", [
    (dict(ht=None), 1), (dict(out=None), 1), (dict(gate=None), 1), (dict(B=0), 2),
    (dict(B=70000), 2), (dict(Hk=7), 3), (dict(dk=129), 4), (dict(dv=126), 4),
    (dict(qks=100), 9), (dict(gbs=47), 9), (dict(io=2), 5), (dict(od=7), 5),
])
def test_step_refusals(lib, kw, status):
    assert step_plan(lib, **kw) == status
    assert "refused" in gdn.last_route()


def test_flag_clear_refuses_null(lib):
    assert lib.gdn_flag_clear(None, None) == 1


def ba_plan(lib, **kw):
    a = dict(x=X, w=X, a_log=X, dt_bias=X, out=X, m=4576, n=96, k=5120, k_stride=5120,
             gate_stride=96, nv=48, G=3, ws=X, ws_bytes=1 << 40)
    a.update(kw)
    return lib.gdn_ba_gates_plan(a["x"], a["w"], a["a_log"], a["dt_bias"], a["out"], a["m"], a["n"],
                                 a["k"], a["k_stride"], a["gate_stride"], a["nv"], a["G"], a["ws"],
                                 a["ws_bytes"])


def test_ba_gates_validation(lib):
    assert ba_plan(lib) == 0
    # 36 tiles of 128 tokens x 7 k splits fill 252 of 256 compute units; 3 compute waves + 1 loader
    assert gdn.last_route().startswith("gdn_ba_partial_kernel+gdn_ba_gate_kernel grid=[36,7,1] block=256")
    assert ba_plan(lib, m=0, x=None, w=None, a_log=None, dt_bias=None, out=None, ws=None, ws_bytes=0) == 0
    assert ba_plan(lib, m=-1) == 2
    assert ba_plan(lib, n=95) == 2                      # n must be 2 nv
    assert ba_plan(lib, nv=47, n=94) == 3               # nv not a multiple of G
    assert ba_plan(lib, nv=66, n=132, G=3) == 4         # n > 128
    assert ba_plan(lib, k=5000, k_stride=5000) == 4     # k not a multiple of 64
    assert ba_plan(lib, k_stride=5100) == 9             # k_stride < k
    assert ba_plan(lib, k_stride=5124) == 9             # not a multiple of 8
    assert ba_plan(lib, gate_stride=95) == 9
    assert ba_plan(lib, m=300000) == 2                  # m * k_stride beyond 2^30
    assert ba_plan(lib, dt_bias=None) == 1
    assert ba_plan(lib, ws=None) == 6
    assert ba_plan(lib, ws_bytes=gdn.gdn_ba_gates_workspace_bytes(4576, 96, 5120) - 1) == 6
    assert "refused" in gdn.last_route()


def test_ba_gates_workspace_size(lib):
    # fp32 partial sums of the k splits (of 64-wide blocks): as many as fill 256 compute
    # units with the 128-token tiles, evened out so that none is empty
    assert gdn.gdn_ba_gates_workspace_bytes(4576, 96, 5120) == 7 * 4576 * 96 * 4
    # one tile: 32 splits of 80 blocks -> 3 blocks each -> 27 splits, none empty
    assert gdn.gdn_ba_gates_workspace_bytes(100, 96, 5120) == 27 * 100 * 96 * 4
    assert gdn.gdn_ba_gates_workspace_bytes(10, 8, 128) == 2 * 10 * 8 * 4
    assert gdn.gdn_ba_gates_workspace_bytes(10, 8, 64) == 1 * 10 * 8 * 4


def test_noalloc_refuses_before_touching_a_device(lib):
    """gdn_chunk_prefill_noalloc validates shapes and its scratch limit on the
    host first: these refusals come back on a machine without a GPU."""
    text = open(HEADER).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gdn.NOALLOC_SCRATCH_BYTES
    big = dict(B=1, T=40000, Hk=16, Hv=48)
    need = gdn.gdn_prefill_workspace_bytes(big["B"], big["T"], big["Hk"], big["Hv"], 128, 128, 64, 1)
    assert need > gdn.NOALLOC_SCRATCH_BYTES
    st = lib.gdn_chunk_prefill_noalloc(X, X, X, X, X, None, X, X, 1, 40000, 16, 48, 128, 128, 64,
                                       None, 1, 1, None)
    assert st == 6, gdn.last_route()
    assert "static scratch" in gdn.last_route()
    st = lib.gdn_chunk_prefill_noalloc(X, X, X, X, X, None, X, X, 1, 128, 16, 47, 128, 128, 64,
                                       None, 1, 1, None)
    assert st == 3   # Hv not a multiple of Hk, refused by the shared validation
    st = lib.gdn_chunk_prefill_noalloc(None, X, X, X, X, None, X, X, 1, 128, 16, 48, 128, 128, 64,
                                       None, 1, 1, None)
    assert st == 1


def test_route_log_once_per_line():
    """GDN_LOG_ROUTE=1 writes each distinct route line to stderr once."""
    import subprocess
    import sys
    code = (
        "import linear_attention_ssm_gated_amd as gdn\n"
        "lib = gdn.library()\n"
        "for T in (128, 128, 256):\n"
        "    lib.gdn_chunk_prefill_plan(1, 1, 1, 1, 1, None, 1, 1, 1, T, 16, 48, 128, 128, 64, None, 1, 1, 1, 1 << 40)\n"
        "lib.gdn_chunk_prefill_plan(1, 1, 1, 1, 1, None, 1, 1, 1, 128, 16, 47, 128, 128, 64, None, 1, 1, 1, 1 << 40)\n"
    )
    env = dict(os.environ, GDN_LOG_ROUTE="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("[gdn route]")]
    assert len(lines) == 2, lines          # one launch route (same geometry for both T) + one refusal
    assert any("refused" in l for l in lines)
    env["GDN_LOG_ROUTE"] = "0"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert "[gdn route]" not in r.stderr
