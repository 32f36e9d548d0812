"""MLA latent-KV decode for MI355X (gfx950): Python binding over libmla.so.

The compute lives in hand-written HIP kernels behind the C ABI declared in
``include/mla.h``; the functions here only marshal torch tensors (device
memory) and the current HIP stream into that ABI.  The native library is
loaded on first use; if it is missing the call raises -- there is no CPU
fallback.  Build it with ``python -m mla_latent_kv_dkv_amd.build``.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_ABI_VERSION = 2
MLA_F32, MLA_BF16 = 0, 1

__all__ = ["MlaDims", "MlaError", "make_dims", "load", "mla_append_latent", "mla_absorb_q",
           "mla_absorb_q_append", "mla_absorb_q_cq", "mla_workspace_bytes_cq",
           "mla_decode_attention", "mla_merge_lse", "mla_absorb_out", "mla_workspace_bytes",
           "mla_append_workspace_bytes", "mla_device_error", "mla_set_kernel_path",
           "mla_status_string", "mla_fp8_page_bytes", "mla_quantize_rows_fp8",
           "mla_append_latent_fp8", "mla_append_workspace_bytes_fp8", "mla_decode_attention_fp8",
           "mla_absorb_q_append_fp8", "mla_absorb_q_append_fp8_workspace_bytes",
           "mla_prefill_attention", "mla_prefill_attention_fp8", "mla_absorb_out_noalloc",
           "mla_absorb_out_noalloc_max_bytes", "mla_decode_plan", "mla_decode_plan_capacity",
           "mla_decode_attention_planned", "mla_decode_attention_fp8_planned",
           "mla_merge_lse_planned", "mla_merge_absorb_out", "mla_merge_absorb_out_workspace_bytes",
           "LIB_PATH"]


class MlaDims(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("rope_scale", ctypes.c_float), ("rope_orig_len", ctypes.c_int32),
                ("yarn_alpha", ctypes.c_float), ("yarn_beta", ctypes.c_float)]


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status}: {mla_status_string(status)}")
        self.status = status


def make_dims(hidden, n_heads, d_head, d_latent, d_rope, dtype="bf16", page_size=64,
              rope_base=10000.0, softmax_scale=0.0, yarn=None) -> MlaDims:
    """``yarn``: None (plain RoPE) or (scale, orig_len, alpha, beta) of YaRN."""
    s, n, a, b = yarn if yarn else (1.0, 0, 0.0, 0.0)
    return MlaDims(MLA_ABI_VERSION, hidden, n_heads, d_head, d_latent, d_rope, page_size,
                   MLA_BF16 if dtype in ("bf16", MLA_BF16) else MLA_F32, rope_base, softmax_scale,
                   s, n, a, b)


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_DIMS = ctypes.POINTER(MlaDims)

_SIGS = {
    "mla_append_latent": [_DIMS, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _P, _I64, _P, _SZ, _P],
    "mla_absorb_q": [_DIMS, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P],
    "mla_absorb_q_append": [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _P, _I64,
                            _P, _P, _P, _SZ, _P],
    "mla_absorb_q_cq": [_DIMS, _I32, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P],
    "mla_decode_attention": [_DIMS, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _P, _P, _P],
    "mla_merge_lse": [_DIMS, _P, _P, _I32, _I32, _P, _P, _P],
    "mla_decode_plan_capacity": [_I32, _I32],
    "mla_decode_plan": [_P, _I32, _I32, _I32, _P, _I64],
    "mla_decode_attention_planned": [_DIMS, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _P, _P,
                                     _P],
    "mla_decode_attention_fp8_planned": [_DIMS, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _P,
                                         _P, _P],
    "mla_merge_lse_planned": [_DIMS, _P, _P, _P, _I32, _I32, _P, _P, _P],
    "mla_absorb_out": [_DIMS, _P, _P, _P, _I32, _P, _P, _SZ, _P],
    "mla_merge_absorb_out": [_DIMS, _P, _P, _I32, _I32, _P, _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "mla_merge_absorb_out_workspace_bytes": [_DIMS, _I32],
    "mla_absorb_out_noalloc": [_DIMS, _P, _P, _P, _I32, _P, _P],
    "mla_absorb_out_noalloc_max_bytes": [],
    "mla_workspace_bytes": [_DIMS, _I32],
    "mla_workspace_bytes_cq": [_DIMS, _I32, _I32],
    "mla_append_workspace_bytes": [_DIMS, _I32],
    "mla_fp8_page_bytes": [_DIMS],
    "mla_quantize_rows_fp8": [_DIMS, _P, _I64, _P, _P, _I32, _P, _I32, _I32, _P, _I64, _P],
    "mla_append_latent_fp8": [_DIMS, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _P, _I64, _P, _SZ,
                              _P],
    "mla_append_workspace_bytes_fp8": [_DIMS, _I32],
    "mla_absorb_q_append_fp8": [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _P,
                                _I64, _P, _P, _P, _SZ, _P],
    "mla_absorb_q_append_fp8_workspace_bytes": [_DIMS, _I32],
    "mla_decode_attention_fp8": [_DIMS, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _P, _P, _P],
    "mla_prefill_attention": [_DIMS, _P, _P, _P, _I64, _P, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _P],
    "mla_prefill_attention_fp8": [_DIMS, _P, _P, _P, _I64, _P, _I32, _I32, _P, _P, _I32, _I32, _P, _P,
                                  _P],
    "mla_status_string": [_I32],
    "mla_abi_version": [],
    "mla_device_error": [ctypes.POINTER(_I32), _I32, _P],
    "mla_set_kernel_path": [_I32],
}
_RES = {"mla_workspace_bytes": _SZ, "mla_workspace_bytes_cq": _SZ, "mla_append_workspace_bytes": _SZ,
        "mla_fp8_page_bytes": _SZ, "mla_append_workspace_bytes_fp8": _SZ,
        "mla_absorb_q_append_fp8_workspace_bytes": _SZ,
        "mla_absorb_out_noalloc_max_bytes": _SZ, "mla_decode_plan_capacity": _I64,
        "mla_merge_absorb_out_workspace_bytes": _SZ,
        "mla_status_string": ctypes.c_char_p}


def load(path: str = LIB_PATH):
    """Load libmla.so (once) and declare its signatures; raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m mla_latent_kv_dkv_amd.build`")
        lib = ctypes.CDLL(path)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _RES.get(name, _I32)
        if lib.mla_abi_version() != MLA_ABI_VERSION:
            raise RuntimeError("libmla.so ABI version mismatch")
        _lib = lib
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to libmla must be contiguous device tensors")
    return _P(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return _P(s.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise MlaError(fn, status)


def _elem(dims: MlaDims):
    import torch
    return torch.bfloat16 if dims.dtype == MLA_BF16 else torch.float32


def _expect(t, shape, dtype, what):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{what}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def mla_status_string(status: int) -> str:
    return load().mla_status_string(status).decode()


def mla_workspace_bytes(dims: MlaDims, batch: int) -> int:
    return int(load().mla_workspace_bytes(ctypes.byref(dims), batch))


def mla_workspace_bytes_cq(dims: MlaDims, d_cq: int, batch: int) -> int:
    return int(load().mla_workspace_bytes_cq(ctypes.byref(dims), d_cq, batch))


def mla_append_workspace_bytes(dims: MlaDims, n_rows: int) -> int:
    return int(load().mla_append_workspace_bytes(ctypes.byref(dims), n_rows))


def mla_set_kernel_path(path: int) -> int:
    return int(load().mla_set_kernel_path(path))


def mla_device_error(clear: bool = True, stream=None) -> int:
    out = _I32(0)
    _check("mla_device_error", load().mla_device_error(ctypes.byref(out), int(clear), _stream(stream)))
    return out.value


def mla_append_latent(dims, h, w_dkv, w_kr, row_seq, row_pos, block_table, pool, workspace=None,
                      stream=None):
    """Write [W_DKV h | RoPE(W_KR h, pos)] of each row of ``h`` into the paged pool.
    ``workspace``: a device byte buffer of at least mla_append_workspace_bytes(dims,
    n_rows) bytes (allocated here when omitted)."""
    import torch
    n, row = h.shape[0], dims.d_latent + dims.d_rope
    _expect(h, (n, dims.hidden), _elem(dims), "h")
    _expect(w_dkv, (dims.d_latent, dims.hidden), _elem(dims), "w_dkv")
    _expect(w_kr, (dims.d_rope, dims.hidden), _elem(dims), "w_kr")
    _expect(row_seq, (n,), torch.int32, "row_seq")
    _expect(row_pos, (n,), torch.int32, "row_pos")
    _expect(pool, (pool.shape[0], dims.page_size, row), _elem(dims), "pool")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be int32 [n_seqs, max_pages]")
    if workspace is None:
        need = mla_append_workspace_bytes(dims, n)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    _check("mla_append_latent", load().mla_append_latent(
        ctypes.byref(dims), _ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(row_seq), _ptr(row_pos), n,
        _ptr(block_table), block_table.shape[0], block_table.shape[1], _ptr(pool), pool.shape[0],
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_absorb_q(dims, h, w_q, w_qr, w_uk, pos, q_lat, q_pe, workspace, stream=None):
    """q_lat = W_UK,i^T W_Q,i h and q_pe = RoPE(W_QR,i h, pos) for every head."""
    import torch
    B, nh = h.shape[0], dims.n_heads
    e = _elem(dims)
    _expect(h, (B, dims.hidden), e, "h")
    _expect(w_q, (nh * dims.d_head, dims.hidden), e, "w_q")
    _expect(w_qr, (nh * dims.d_rope, dims.hidden), e, "w_qr")
    _expect(w_uk, (nh * dims.d_head, dims.d_latent), e, "w_uk")
    _expect(pos, (B,), torch.int32, "pos")
    _expect(q_lat, (B, nh, dims.d_latent), torch.float32, "q_lat")
    _expect(q_pe, (B, nh, dims.d_rope), torch.float32, "q_pe")
    _check("mla_absorb_q", load().mla_absorb_q(
        ctypes.byref(dims), _ptr(h), _ptr(w_q), _ptr(w_qr), _ptr(w_uk), _ptr(pos), B, _ptr(q_lat),
        _ptr(q_pe), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_absorb_q_append(dims, h, w_q, w_qr, w_uk, w_dkv, w_kr, pos, row_seq, block_table, pool,
                        q_lat, q_pe, workspace, stream=None):
    """mla_absorb_q and mla_append_latent of the same rows (row b = token
    (row_seq[b], pos[b])) in one call; one projection over all four weights
    where the matrix-core path applies."""
    import torch
    B, nh, row = h.shape[0], dims.n_heads, dims.d_latent + dims.d_rope
    e = _elem(dims)
    _expect(h, (B, dims.hidden), e, "h")
    _expect(w_q, (nh * dims.d_head, dims.hidden), e, "w_q")
    _expect(w_qr, (nh * dims.d_rope, dims.hidden), e, "w_qr")
    _expect(w_uk, (nh * dims.d_head, dims.d_latent), e, "w_uk")
    _expect(w_dkv, (dims.d_latent, dims.hidden), e, "w_dkv")
    _expect(w_kr, (dims.d_rope, dims.hidden), e, "w_kr")
    _expect(pos, (B,), torch.int32, "pos")
    _expect(row_seq, (B,), torch.int32, "row_seq")
    _expect(pool, (pool.shape[0], dims.page_size, row), e, "pool")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be int32 [n_seqs, max_pages]")
    _expect(q_lat, (B, nh, dims.d_latent), torch.float32, "q_lat")
    _expect(q_pe, (B, nh, dims.d_rope), torch.float32, "q_pe")
    _check("mla_absorb_q_append", load().mla_absorb_q_append(
        ctypes.byref(dims), _ptr(h), _ptr(w_q), _ptr(w_qr), _ptr(w_uk), _ptr(w_dkv), _ptr(w_kr),
        _ptr(pos), _ptr(row_seq), B, _ptr(block_table), block_table.shape[0], block_table.shape[1],
        _ptr(pool), pool.shape[0], _ptr(q_lat), _ptr(q_pe), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_absorb_q_cq(dims, h, w_dq, w_uq, w_qr, w_uk, pos, q_lat, q_pe, workspace, stream=None):
    """q_lat = W_UK,i^T W_UQ,i W_DQ h and q_pe = RoPE(W_QR,i h, pos) for every head
    (query low-rank compression; d_cq = w_dq.shape[0])."""
    import torch
    B, nh = h.shape[0], dims.n_heads
    e = _elem(dims)
    d_cq = w_dq.shape[0]
    _expect(h, (B, dims.hidden), e, "h")
    _expect(w_dq, (d_cq, dims.hidden), e, "w_dq")
    _expect(w_uq, (nh * dims.d_head, d_cq), e, "w_uq")
    _expect(w_qr, (nh * dims.d_rope, dims.hidden), e, "w_qr")
    _expect(w_uk, (nh * dims.d_head, dims.d_latent), e, "w_uk")
    _expect(pos, (B,), torch.int32, "pos")
    _expect(q_lat, (B, nh, dims.d_latent), torch.float32, "q_lat")
    _expect(q_pe, (B, nh, dims.d_rope), torch.float32, "q_pe")
    _check("mla_absorb_q_cq", load().mla_absorb_q_cq(
        ctypes.byref(dims), d_cq, _ptr(h), _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), _ptr(w_uk),
        _ptr(pos), B, _ptr(q_lat), _ptr(q_pe), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_decode_attention(dims, q_lat, q_pe, pool, block_table, seq_lens, o_part, lse_part,
                         stream=None):
    """Split-KV latent attention; the split count is o_part.shape[1]."""
    import torch
    B, S = o_part.shape[0], o_part.shape[1]
    nh, e = dims.n_heads, _elem(dims)
    _expect(q_lat, (B, nh, dims.d_latent), torch.float32, "q_lat")
    _expect(q_pe, (B, nh, dims.d_rope), torch.float32, "q_pe")
    _expect(pool, (pool.shape[0], dims.page_size, dims.d_latent + dims.d_rope), e, "pool")
    _expect(seq_lens, (B,), torch.int32, "seq_lens")
    _expect(o_part, (B, S, nh, dims.d_latent), torch.float32, "o_part")
    _expect(lse_part, (B, S, nh), torch.float32, "lse_part")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] < B:
        raise ValueError("block_table must be int32 [>= batch, max_pages]")
    _check("mla_decode_attention", load().mla_decode_attention(
        ctypes.byref(dims), _ptr(q_lat), _ptr(q_pe), _ptr(pool), pool.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), B, S, _ptr(o_part), _ptr(lse_part), _stream(stream)))


def mla_merge_lse(dims, o_part, lse_part, o_lat, lse=None, stream=None):
    """Log-sum-exp merge of the split partials into o_lat (and lse if given)."""
    import torch
    B, S = o_part.shape[0], o_part.shape[1]
    nh = dims.n_heads
    _expect(o_part, (B, S, nh, dims.d_latent), torch.float32, "o_part")
    _expect(lse_part, (B, S, nh), torch.float32, "lse_part")
    _expect(o_lat, (B, nh, dims.d_latent), torch.float32, "o_lat")
    if lse is not None:
        _expect(lse, (B, nh), torch.float32, "lse")
    _check("mla_merge_lse", load().mla_merge_lse(
        ctypes.byref(dims), _ptr(o_part), _ptr(lse_part), B, S, _ptr(o_lat), _ptr(lse),
        _stream(stream)))


def mla_decode_plan_capacity(batch: int, target_units: int) -> int:
    return int(load().mla_decode_plan_capacity(batch, target_units))


def mla_decode_plan(seq_lens, page_size: int, target_units: int):
    """Length-proportional work list (host): returns (n_units, plan) with plan an
    int32 numpy array of 3 n_units unit entries followed by batch + 1 unit starts."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    cap = mla_decode_plan_capacity(len(lens), target_units)
    if cap <= 0:
        raise ValueError("batch or target_units out of range")
    plan = np.zeros(cap, dtype=np.int32)
    n = int(load().mla_decode_plan(lens.ctypes.data_as(_P), len(lens), page_size, target_units,
                                   plan.ctypes.data_as(_P), cap))
    if n < 0:
        raise MlaError("mla_decode_plan", n)
    return n, plan[:3 * n + len(lens) + 1].copy()


def _attention_planned(name, fp8, dims, q_lat, q_pe, pool, block_table, plan, n_units, o_part,
                       lse_part, stream):
    import torch
    B, nh = q_lat.shape[0], dims.n_heads
    _expect(q_lat, (B, nh, dims.d_latent), torch.float32, "q_lat")
    _expect(q_pe, (B, nh, dims.d_rope), torch.float32, "q_pe")
    if fp8:
        _expect_fp8_pool(dims, pool)
    else:
        _expect(pool, (pool.shape[0], dims.page_size, dims.d_latent + dims.d_rope), _elem(dims),
                "pool")
    _expect(plan, (3 * n_units + B + 1,), torch.int32, "plan")
    _expect(o_part, (n_units, nh, dims.d_latent), torch.float32, "o_part")
    _expect(lse_part, (n_units, nh), torch.float32, "lse_part")
    _expect_table(block_table)
    if block_table.shape[0] < B:
        raise ValueError("block_table must have at least batch rows")
    _check(name, getattr(load(), name)(
        ctypes.byref(dims), _ptr(q_lat), _ptr(q_pe), _ptr(pool), pool.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(plan), n_units, B, _ptr(o_part), _ptr(lse_part),
        _stream(stream)))


def mla_decode_attention_planned(dims, q_lat, q_pe, pool, block_table, plan, n_units, o_part,
                                 lse_part, stream=None):
    """Split-KV latent attention over the units of a plan (device int32 copy of
    mla_decode_plan's array)."""
    _attention_planned("mla_decode_attention_planned", False, dims, q_lat, q_pe, pool,
                       block_table, plan, n_units, o_part, lse_part, stream)


def mla_decode_attention_fp8_planned(dims, q_lat, q_pe, pool, block_table, plan, n_units, o_part,
                                     lse_part, stream=None):
    """mla_decode_attention_planned over the FP8 pool."""
    _attention_planned("mla_decode_attention_fp8_planned", True, dims, q_lat, q_pe, pool,
                       block_table, plan, n_units, o_part, lse_part, stream)


def mla_merge_lse_planned(dims, o_part, lse_part, plan, n_units, o_lat, lse=None, stream=None):
    """Log-sum-exp merge of a plan's unit partials into o_lat (and lse if given)."""
    import torch
    B, nh = o_lat.shape[0], dims.n_heads
    _expect(o_part, (n_units, nh, dims.d_latent), torch.float32, "o_part")
    _expect(lse_part, (n_units, nh), torch.float32, "lse_part")
    _expect(plan, (3 * n_units + B + 1,), torch.int32, "plan")
    _expect(o_lat, (B, nh, dims.d_latent), torch.float32, "o_lat")
    if lse is not None:
        _expect(lse, (B, nh), torch.float32, "lse")
    _check("mla_merge_lse_planned", load().mla_merge_lse_planned(
        ctypes.byref(dims), _ptr(o_part), _ptr(lse_part), _ptr(plan), n_units, B, _ptr(o_lat),
        _ptr(lse), _stream(stream)))


def mla_absorb_out(dims, o_lat, w_uv, w_o, u, workspace, stream=None):
    """u = W_O [W_UV,i o_lat,i]_i."""
    import torch
    B, nh, e = o_lat.shape[0], dims.n_heads, _elem(dims)
    _expect(o_lat, (B, nh, dims.d_latent), torch.float32, "o_lat")
    _expect(w_uv, (nh * dims.d_head, dims.d_latent), e, "w_uv")
    _expect(w_o, (dims.hidden, nh * dims.d_head), e, "w_o")
    _expect(u, (B, dims.hidden), torch.float32, "u")
    _check("mla_absorb_out", load().mla_absorb_out(
        ctypes.byref(dims), _ptr(o_lat), _ptr(w_uv), _ptr(w_o), B, _ptr(u), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_merge_absorb_out_workspace_bytes(dims: MlaDims, batch: int) -> int:
    return int(load().mla_merge_absorb_out_workspace_bytes(ctypes.byref(dims), batch))


def mla_merge_absorb_out(dims, o_part, lse_part, w_uv, w_o, u, workspace, lse=None, plan=None,
                         n_units=0, stream=None):
    """mla_merge_lse (uniform splits: o_part [B, S, n_h, d_c]; or over a plan:
    o_part [n_units, n_h, d_c]) then mla_absorb_out, in one call: u, and lse if given."""
    import torch
    B, nh, e = u.shape[0], dims.n_heads, _elem(dims)
    if plan is None:
        S = o_part.shape[1]
        _expect(o_part, (B, S, nh, dims.d_latent), torch.float32, "o_part")
        _expect(lse_part, (B, S, nh), torch.float32, "lse_part")
    else:
        S = 1
        _expect(o_part, (n_units, nh, dims.d_latent), torch.float32, "o_part")
        _expect(lse_part, (n_units, nh), torch.float32, "lse_part")
        _expect(plan, (3 * n_units + B + 1,), torch.int32, "plan")
    _expect(w_uv, (nh * dims.d_head, dims.d_latent), e, "w_uv")
    _expect(w_o, (dims.hidden, nh * dims.d_head), e, "w_o")
    _expect(u, (B, dims.hidden), torch.float32, "u")
    if lse is not None:
        _expect(lse, (B, nh), torch.float32, "lse")
    _check("mla_merge_absorb_out", load().mla_merge_absorb_out(
        ctypes.byref(dims), _ptr(o_part), _ptr(lse_part), B, S, _ptr(plan), n_units, _ptr(w_uv),
        _ptr(w_o), _ptr(u), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_absorb_out_noalloc(dims, o_lat, w_uv, w_o, u, stream=None):
    """mla_absorb_out with the library's static scratch instead of a workspace
    (nothing is allocated; calls overlapping on one device race)."""
    import torch
    B, nh, e = o_lat.shape[0], dims.n_heads, _elem(dims)
    _expect(o_lat, (B, nh, dims.d_latent), torch.float32, "o_lat")
    _expect(w_uv, (nh * dims.d_head, dims.d_latent), e, "w_uv")
    _expect(w_o, (dims.hidden, nh * dims.d_head), e, "w_o")
    _expect(u, (B, dims.hidden), torch.float32, "u")
    _check("mla_absorb_out_noalloc", load().mla_absorb_out_noalloc(
        ctypes.byref(dims), _ptr(o_lat), _ptr(w_uv), _ptr(w_o), B, _ptr(u), _stream(stream)))


def mla_absorb_out_noalloc_max_bytes() -> int:
    return int(load().mla_absorb_out_noalloc_max_bytes())


# ------------------------------------------------------------- FP8 pool --
def mla_fp8_page_bytes(dims: MlaDims) -> int:
    return int(load().mla_fp8_page_bytes(ctypes.byref(dims)))


def mla_append_workspace_bytes_fp8(dims: MlaDims, n_rows: int) -> int:
    return int(load().mla_append_workspace_bytes_fp8(ctypes.byref(dims), n_rows))


def _expect_fp8_pool(dims, pool):
    import torch
    pb = mla_fp8_page_bytes(dims)
    if pool.dtype != torch.uint8 or pool.dim() != 2 or pool.shape[1] != pb:
        raise ValueError(f"FP8 pool must be uint8 [num_pages, {pb}], got "
                         f"{tuple(pool.shape)} {pool.dtype}")


def _expect_table(block_table):
    import torch
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be int32 [n_seqs, max_pages]")


def mla_quantize_rows_fp8(dims, rows, row_seq, row_pos, block_table, pool, stream=None):
    """Quantize fp32 rows [n, >= d_c + d_R] ([c | k^R], k^R already rotated) into
    their slots of the FP8 pool (uint8 [num_pages, mla_fp8_page_bytes(dims)])."""
    import torch
    n = rows.shape[0]
    if rows.dtype != torch.float32 or rows.dim() != 2 or rows.shape[1] < dims.d_latent + dims.d_rope:
        raise ValueError("rows must be fp32 [n, >= d_c + d_R]")
    _expect(row_seq, (n,), torch.int32, "row_seq")
    _expect(row_pos, (n,), torch.int32, "row_pos")
    _expect_table(block_table)
    _expect_fp8_pool(dims, pool)
    _check("mla_quantize_rows_fp8", load().mla_quantize_rows_fp8(
        ctypes.byref(dims), _ptr(rows), rows.shape[1], _ptr(row_seq), _ptr(row_pos), n,
        _ptr(block_table), block_table.shape[0], block_table.shape[1], _ptr(pool), pool.shape[0],
        _stream(stream)))


def mla_append_latent_fp8(dims, h, w_dkv, w_kr, row_seq, row_pos, block_table, pool,
                          workspace=None, stream=None):
    """mla_append_latent into the FP8 pool: rows in fp32, k^R rotated, then quantized.
    ``workspace``: at least mla_append_workspace_bytes_fp8(dims, n_rows) bytes
    (allocated here when omitted)."""
    import torch
    n = h.shape[0]
    _expect(h, (n, dims.hidden), _elem(dims), "h")
    _expect(w_dkv, (dims.d_latent, dims.hidden), _elem(dims), "w_dkv")
    _expect(w_kr, (dims.d_rope, dims.hidden), _elem(dims), "w_kr")
    _expect(row_seq, (n,), torch.int32, "row_seq")
    _expect(row_pos, (n,), torch.int32, "row_pos")
    _expect_table(block_table)
    _expect_fp8_pool(dims, pool)
    if workspace is None:
        need = mla_append_workspace_bytes_fp8(dims, n)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    _check("mla_append_latent_fp8", load().mla_append_latent_fp8(
        ctypes.byref(dims), _ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(row_seq), _ptr(row_pos), n,
        _ptr(block_table), block_table.shape[0], block_table.shape[1], _ptr(pool), pool.shape[0],
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_absorb_q_append_fp8_workspace_bytes(dims: MlaDims, batch: int) -> int:
    return int(load().mla_absorb_q_append_fp8_workspace_bytes(ctypes.byref(dims), batch))


def mla_absorb_q_append_fp8(dims, h, w_q, w_qr, w_uk, w_dkv, w_kr, pos, row_seq, block_table,
                            pool, q_lat, q_pe, workspace, stream=None):
    """mla_absorb_q and mla_append_latent_fp8 of the same rows (row b = token
    (row_seq[b], pos[b])) in one call; one projection over all four weights where
    the matrix-core path applies.  ``workspace``: at least
    mla_absorb_q_append_fp8_workspace_bytes(dims, batch) bytes."""
    import torch
    B, nh = h.shape[0], dims.n_heads
    e = _elem(dims)
    _expect(h, (B, dims.hidden), e, "h")
    _expect(w_q, (nh * dims.d_head, dims.hidden), e, "w_q")
    _expect(w_qr, (nh * dims.d_rope, dims.hidden), e, "w_qr")
    _expect(w_uk, (nh * dims.d_head, dims.d_latent), e, "w_uk")
    _expect(w_dkv, (dims.d_latent, dims.hidden), e, "w_dkv")
    _expect(w_kr, (dims.d_rope, dims.hidden), e, "w_kr")
    _expect(pos, (B,), torch.int32, "pos")
    _expect(row_seq, (B,), torch.int32, "row_seq")
    _expect_table(block_table)
    _expect_fp8_pool(dims, pool)
    _expect(q_lat, (B, nh, dims.d_latent), torch.float32, "q_lat")
    _expect(q_pe, (B, nh, dims.d_rope), torch.float32, "q_pe")
    _check("mla_absorb_q_append_fp8", load().mla_absorb_q_append_fp8(
        ctypes.byref(dims), _ptr(h), _ptr(w_q), _ptr(w_qr), _ptr(w_uk), _ptr(w_dkv), _ptr(w_kr),
        _ptr(pos), _ptr(row_seq), B, _ptr(block_table), block_table.shape[0], block_table.shape[1],
        _ptr(pool), pool.shape[0], _ptr(q_lat), _ptr(q_pe), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_decode_attention_fp8(dims, q_lat, q_pe, pool, block_table, seq_lens, o_part, lse_part,
                             stream=None):
    """Split-KV latent attention over the FP8 pool; the split count is o_part.shape[1]."""
    import torch
    B, S = o_part.shape[0], o_part.shape[1]
    nh = dims.n_heads
    _expect(q_lat, (B, nh, dims.d_latent), torch.float32, "q_lat")
    _expect(q_pe, (B, nh, dims.d_rope), torch.float32, "q_pe")
    _expect_fp8_pool(dims, pool)
    _expect(seq_lens, (B,), torch.int32, "seq_lens")
    _expect(o_part, (B, S, nh, dims.d_latent), torch.float32, "o_part")
    _expect(lse_part, (B, S, nh), torch.float32, "lse_part")
    _expect_table(block_table)
    if block_table.shape[0] < B:
        raise ValueError("block_table must have at least batch rows")
    _check("mla_decode_attention_fp8", load().mla_decode_attention_fp8(
        ctypes.byref(dims), _ptr(q_lat), _ptr(q_pe), _ptr(pool), pool.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), B, S, _ptr(o_part), _ptr(lse_part), _stream(stream)))


# -------------------------------------------------------------- prefill --
def mla_prefill_attention(dims, q_lat, q_pe, pool, block_table, q_seq, q_pos, o_part, lse_part,
                          stream=None, fp8=False):
    """Causal attention of query tokens (q_seq[i], q_pos[i]) over their sequences'
    cached rows 0..q_pos[i]; the split count is o_part.shape[1].  ``fp8``: the pool
    is an FP8 pool (uint8 [num_pages, mla_fp8_page_bytes(dims)])."""
    import torch
    n, S = o_part.shape[0], o_part.shape[1]
    nh = dims.n_heads
    _expect(q_lat, (n, nh, dims.d_latent), torch.float32, "q_lat")
    _expect(q_pe, (n, nh, dims.d_rope), torch.float32, "q_pe")
    if fp8:
        _expect_fp8_pool(dims, pool)
    else:
        _expect(pool, (pool.shape[0], dims.page_size, dims.d_latent + dims.d_rope), _elem(dims), "pool")
    _expect(q_seq, (n,), torch.int32, "q_seq")
    _expect(q_pos, (n,), torch.int32, "q_pos")
    _expect(o_part, (n, S, nh, dims.d_latent), torch.float32, "o_part")
    _expect(lse_part, (n, S, nh), torch.float32, "lse_part")
    _expect_table(block_table)
    fn = "mla_prefill_attention_fp8" if fp8 else "mla_prefill_attention"
    _check(fn, getattr(load(), fn)(
        ctypes.byref(dims), _ptr(q_lat), _ptr(q_pe), _ptr(pool), pool.shape[0], _ptr(block_table),
        block_table.shape[0], block_table.shape[1], _ptr(q_seq), _ptr(q_pos), n, S, _ptr(o_part),
        _ptr(lse_part), _stream(stream)))


def mla_prefill_attention_fp8(dims, q_lat, q_pe, pool, block_table, q_seq, q_pos, o_part, lse_part,
                              stream=None):
    mla_prefill_attention(dims, q_lat, q_pe, pool, block_table, q_seq, q_pos, o_part, lse_part,
                          stream, fp8=True)


def default_scale(dims: MlaDims) -> float:
    """tau as the library takes it from ``dims`` (YaRN's logit factor included)."""
    tau = dims.softmax_scale if dims.softmax_scale > 0 else 1.0 / math.sqrt(dims.d_head + dims.d_rope)
    if dims.rope_scale > 1.0:
        tau *= (0.1 * math.log(dims.rope_scale) + 1.0) ** 2
    return tau
