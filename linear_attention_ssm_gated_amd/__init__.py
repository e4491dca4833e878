"""Python binding of libgdn.so, the gfx950 gated delta rule library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/gdn.h).  PyTorch supplies device memory and
the current stream.  The functions named like the C entry points take torch
tensors and pass their device pointers through; there is no fallback: if the
library is not built, or a call is refused, an exception says so.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_F32 = 0
GDN_BF16 = 1
K_ROWS = 4
NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h

_STATUS = {
    0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_HEAD_GROUPS",
    4: "GDN_ERR_DIM_LIMIT", 5: "GDN_ERR_DTYPE", 6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_STASH",
    8: "GDN_ERR_K_ROWS", 9: "GDN_ERR_STRIDE", 10: "GDN_ERR_SLABS", 11: "GDN_ERR_HIP",
}

# name -> (restype, argtypes) of every entry point include/gdn.h declares
P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "gdn_status_string": (ctypes.c_char_p, [I]),
    "gdn_last_route": (ctypes.c_char_p, []),
    "gdn_prefill_workspace_bytes": (Z, [I, I, I, I, I, I, I, I, I]),
    "gdn_chunk_prefill": (I, [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, I, I, P, Z, P]),
    "gdn_chunk_prefill_plan": (I, [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, I, I, P, Z]),
    "gdn_chunk_prefill_segmented": (I, [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, I, I, P, Z, P]),
    "gdn_chunk_prefill_segmented_plan": (I, [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, I, I, P, Z]),
    "gdn_chunk_prefill_noalloc": (I, [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, I, I, P]),
    "gdn_stash_seq_floats": (Z, [I, I, I, I, I]),
    "gdn_flag_clear": (I, [P, P]),
    "gdn_decode_verify": (I, [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P, I, I, P]),
    "gdn_decode_verify_plan": (I, [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P, I, I]),
    "gdn_decode_verify_k4": (I, [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, I, I, P]),
    "gdn_decode_verify_k4_plan": (I, [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, I, I]),
    "gdn_decode_verify_parent": (I, [P, P, I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, I, I, P]),
    "gdn_decode_verify_parent_plan": (I, [P, P, I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, I, I]),
    "gdn_fold": (I, [P, P, P, P, I, P, I, I, I, I, I, I, I, I, P]),
    "gdn_fold_plan": (I, [P, P, P, P, I, P, I, I, I, I, I, I, I, I]),
    "gdn_decode_step": (I, [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P]),
    "gdn_decode_step_plan": (I, [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I]),
    "gdn_ba_gates_workspace_bytes": (Z, [I, I, I]),
    "gdn_ba_gates": (I, [P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]),
    "gdn_ba_gates_plan": (I, [P, P, P, P, P, I, I, I, I, I, I, I, P, Z]),
}

_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int, route: str):
        super().__init__(f"{_STATUS.get(status, status)}: {route}")
        self.status = status
        self.route = route


def library():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def last_route() -> str:
    return library().gdn_last_route().decode()


def status_string(status: int) -> str:
    return library().gdn_status_string(status).decode()


def _check(status: int):
    if status != 0:
        raise GdnError(status, last_route())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ---- entry points, same names as the C ABI --------------------------------

def gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, io_dtype, packed=False) -> int:
    return library().gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, io_dtype, int(bool(packed)))


def gdn_chunk_prefill(q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv, chunk,
                      cu_seqlens=None, workspace=None, stream=None):
    """Enqueue one chunked prefill (layouts in include/gdn.h).  Returns the route line."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().gdn_chunk_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta), _ptr(h0), _ptr(out), _ptr(h_final),
        B, T, Hk, Hv, dk, dv, chunk, _ptr(cu_seqlens), _dtype_code(q), _dtype_code(out),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return last_route()


def gdn_chunk_prefill_segmented(q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv, chunk,
                                cu_seqlens=None, workspace=None, stream=None):
    """Enqueue one segment-scan prefill (include/gdn.h).  Returns the route line."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().gdn_chunk_prefill_segmented(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta), _ptr(h0), _ptr(out), _ptr(h_final),
        B, T, Hk, Hv, dk, dv, chunk, _ptr(cu_seqlens), _dtype_code(q), _dtype_code(out),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return last_route()


def gdn_chunk_prefill_noalloc(q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv, chunk,
                              cu_seqlens=None, stream=None):
    """gdn_chunk_prefill with the library's static device scratch (no workspace,
    no allocation).  Returns the route line."""
    _check(library().gdn_chunk_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta), _ptr(h0), _ptr(out), _ptr(h_final),
        B, T, Hk, Hv, dk, dv, chunk, _ptr(cu_seqlens), _dtype_code(q), _dtype_code(out),
        _stream(stream)))
    return last_route()


def gdn_stash_seq_floats(Hv, dk, dv, k_rows=K_ROWS, io_dtype=GDN_BF16) -> int:
    return library().gdn_stash_seq_floats(Hv, dk, dv, k_rows, io_dtype)


def gdn_flag_clear(engaged_flag, stream=None):
    _check(library().gdn_flag_clear(_ptr(engaged_flag), _stream(stream)))


def gdn_decode_verify_k4(h_table, q, k, v, gate, beta, out, stash, B, Hk, Hv, dk, dv,
                         qk_stride, v_stride, gb_stride, stash_seq_floats, engaged_flag,
                         stream=None):
    _check(library().gdn_decode_verify_k4(
        _ptr(h_table), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(out), _ptr(stash),
        B, Hk, Hv, dk, dv, qk_stride, v_stride, gb_stride, stash_seq_floats, _ptr(engaged_flag),
        _dtype_code(q), _dtype_code(out), _stream(stream)))
    return last_route()


def gdn_decode_verify(h_table, q, k, v, gate, beta, out, stash, B, Hk, Hv, dk, dv, k_rows,
                      qk_stride, v_stride, gb_stride, stash_seq_floats, engaged_flag, stream=None):
    _check(library().gdn_decode_verify(
        _ptr(h_table), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(out), _ptr(stash),
        B, Hk, Hv, dk, dv, k_rows, qk_stride, v_stride, gb_stride, stash_seq_floats,
        _ptr(engaged_flag), _dtype_code(q), _dtype_code(out), _stream(stream)))
    return last_route()


def gdn_decode_verify_parent(h_table, hi_tables, slab_entries, q, k, v, gate, beta, out, stash, B, Hk,
                             Hv, dk, dv, k_rows, qk_stride, v_stride, gb_stride, stash_seq_floats,
                             stream=None):
    _check(library().gdn_decode_verify_parent(
        _ptr(h_table), _ptr(hi_tables), slab_entries, _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
        _ptr(beta), _ptr(out), _ptr(stash), B, Hk, Hv, dk, dv, k_rows, qk_stride, v_stride,
        gb_stride, stash_seq_floats, _dtype_code(q), _dtype_code(out), _stream(stream)))
    return last_route()


def gdn_decode_step(h_table, q, k, v, gate, beta, out, B, Hk, Hv, dk, dv, qk_stride, v_stride,
                    gb_stride, stream=None):
    _check(library().gdn_decode_step(
        _ptr(h_table), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(out), B, Hk, Hv,
        dk, dv, qk_stride, v_stride, gb_stride, _dtype_code(q), _dtype_code(out), _stream(stream)))
    return last_route()


def gdn_fold(h_table, stash, na_tab, hi_tables, slab_entries, engaged_flag, k_rows, B, Hk, Hv,
             dk, dv, stash_seq_floats, io_dtype, stream=None):
    _check(library().gdn_fold(
        _ptr(h_table), _ptr(stash), _ptr(na_tab), _ptr(hi_tables), slab_entries,
        _ptr(engaged_flag), k_rows, B, Hk, Hv, dk, dv, stash_seq_floats, io_dtype,
        _stream(stream)))
    return last_route()


# ---- allocation conveniences (torch allocates, the library computes) ------

def gdn_ba_gates_workspace_bytes(m, n, k) -> int:
    return library().gdn_ba_gates_workspace_bytes(m, n, k)


def gdn_ba_gates(input, ba_weight, a_log, dt_bias, gate_out, m, n, k, k_stride, gate_stride, nv,
                 vheads_per_group, workspace=None, stream=None):
    """Enqueue one gate/beta producer call (layouts in include/gdn.h).  Returns the route line."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().gdn_ba_gates(
        _ptr(input), _ptr(ba_weight), _ptr(a_log), _ptr(dt_bias), _ptr(gate_out), m, n, k, k_stride,
        gate_stride, nv, vheads_per_group, _ptr(workspace), ws_bytes, _stream(stream)))
    return last_route()


def ba_gates(x, w, a_log, dt_bias, nv, vheads_per_group, gate_stride=None, stream=None):
    """Allocate the output and workspace with torch and run gdn_ba_gates.

    x: bf16 [m, k_stride] (the first k = w.shape[1] columns used); w: bf16
    [2 nv, k]; a_log, dt_bias: fp32 [nv].  Returns (gate_out fp32 [m,
    gate_stride] with the gates in columns 0..nv-1 and beta in nv..2nv-1,
    route line).
    """
    m, k_stride = x.shape
    n, k = w.shape
    gs = 2 * nv if gate_stride is None else gate_stride
    out = torch.empty((m, gs), dtype=torch.float32, device=x.device)
    ws_n = gdn_ba_gates_workspace_bytes(m, n, k)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=x.device) if ws_n else None
    route = gdn_ba_gates(x, w, a_log, dt_bias, out, m, n, k, k_stride, gs, nv, vheads_per_group,
                         workspace=ws, stream=stream)
    return out, route


def chunk_prefill(q, k, v, log_g, beta, h0=None, cu_seqlens=None, chunk=64, out_dtype=None,
                  want_state=True, stream=None, segmented=False):
    """Allocate out/h_final with torch and run gdn_chunk_prefill (or, with
    segmented=True, gdn_chunk_prefill_segmented).

    Dense q, k [B, T, Hk, dk], v [B, T, Hv, dv], log_g/beta [B, T, Hv]; or
    packed q, k [N, Hk, dk] ... with cu_seqlens [B+1] (int32, on the GPU).
    Returns (out, h_final or None, route line).
    """
    if cu_seqlens is not None:
        B = cu_seqlens.numel() - 1
        T, Hk, dk = q.shape
    else:
        B, T, Hk, dk = q.shape
    Hv, dv = v.shape[-2], v.shape[-1]
    out = torch.empty(v.shape, dtype=out_dtype or v.dtype, device=v.device)
    hf = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=v.device) if want_state else None
    ws_n = gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, _dtype_code(q),
                                       packed=cu_seqlens is not None)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=v.device) if ws_n else None
    call = gdn_chunk_prefill_segmented if segmented else gdn_chunk_prefill
    route = call(q, k, v, log_g, beta, h0, out, hf, B, T, Hk, Hv, dk, dv, chunk,
                 cu_seqlens=cu_seqlens, workspace=ws, stream=stream)
    return out, hf, route
